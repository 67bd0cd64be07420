// Read path (unified_attention_int4) on the matrix cores: paged attention
// over the int4 RHT cache where the query block is dense -- the query heads
// of one GQA group and/or several query tokens of a prefill chunk share every
// K/V element they read.
//
// Math per query row, as in the vector-ALU kernel (vLLM PR #62881 "[Bugfix]
// [Test] Rotate KV into RHT domain in the INT4 unified attn test", Details /
// Root cause; divisor b per runguoli.com "vLLM -- Attention Kernels & KV
// Cache Quantization", section "PR #56198"): q' = H.D.q, logit_j = k_scale_j
// (q' . code_j) softmax_scale / b, online softmax, o' = sum p_j v_scale_j
// code_V_j, out = D.H.o'/b.
//
// gfx950 mapping. One wave = one work unit (sequence, query tile of up to 16
// rows -- 32 with two row blocks --, group of hpw kv heads, KV range: a split,
// or a stream-K piece in decode); a workgroup takes consecutive units
// (neighbouring kv heads of the same pages, whose code rows share cache lines
// inside one CU). The KV range is walked 32 tokens (two 16-token half tiles)
// per step, with the loads of the next step in flight (direct buffer->LDS
// loads into two stage slots):
//   * S^T = K . Q'^T on v_mfma_f32_16x16x32_bf16: A = K codes (16 tokens x 32
//     head elements), B = q' rows (bf16). The head dimension is permuted so
//     that a lane's 16 / 12 / 8 ... code bytes of one token are one vector
//     load and feed all k-steps; q' is permuted the same way. q' enters as a
//     bf16 hi + lo pair (two MFMAs), ~16 significant bits: sharp softmax rows
//     (large k_scale from outlier channels) stay within 1e-2 of the fp64
//     result.
//   * K codes become bf16 operands exactly, two per VALU op: (u & 0xF) |
//     0x4300 is the bf16 of 128 + u with u = code + 8 (nibble xor 8); the
//     constant 136 is removed after the product with the sum of q'.
//   * The S^T accumulator leaves each lane with 8 logits of ONE query row,
//     which is exactly the B-operand layout P^T needs for O'^T = V^T P^T, so
//     softmax runs in registers with no transpose; the V^T operand is built
//     from 8 tokens' code words per lane (byte permutes + masks).
//   * O'^T = V^T P^T on v_mfma_f32_16x16x32_f16: V codes become the fp16 of
//     64 + u exactly; p * v_scale is one fp16 (11 significant bits) under a
//     per-step power-of-two scale that bounds it (see the softmax step). The
//     constant 72 is removed with the sum of the rounded P, taken by one
//     extra MFMA against a ones operand.
//   * k_scale / v_scale of the 32 tokens are loaded once per step (one lane
//     per token) and redistributed through a 256-byte LDS slot per head.
// Pages are looked up once per 16-token half tile (block_size % 16 == 0).
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <unordered_map>
#include <type_traits>

#include "kv4_device.hpp"
#include "kv4_launch.hpp"
#include "kv4_mfma_ops.hpp"

namespace kv4 {


// ---- one-byte codes of the per-token-head int8 / fp8 caches -> fp16 pairs
// (exact). int8: the fp16 of 1024 + (code + 128) = 1152 + code, i.e. the
// offset byte under the exponent of 1024; fp8 e4m3fn: v_cvt_scalef32_pk_f16_fp8
// with unit scale (every finite e4m3 value, subnormals included, is an fp16).
typedef _Float16 f16x2v_t __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// 8 consecutive codes (two words) of one token -> A operand of one k-step,
// natural element order.
template <int QM>
__device__ __forceinline__ uint4 k_operand_q(uint32_t w0, uint32_t w1) {
  if constexpr (QM == 1) {
    const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
    const uint32_t c = 0x64646464u;
    return make_uint4(__builtin_amdgcn_perm(c, x0, 0x04010400u), __builtin_amdgcn_perm(c, x0, 0x04030402u),
                      __builtin_amdgcn_perm(c, x1, 0x04010400u), __builtin_amdgcn_perm(c, x1, 0x04030402u));
  } else {
    return make_uint4(fp8x2_to_f16x2<false>(w0), fp8x2_to_f16x2<true>(w0), fp8x2_to_f16x2<false>(w1),
                      fp8x2_to_f16x2<true>(w1));
  }
}

// V^T operands of columns jb and jb + 1 of a lane's 4-column word from 8
// token words x[0..7] (token order = k order).
template <int QM>
__device__ __forceinline__ void v_operands_q(const uint32_t (&x)[8], int jb, uint4& c0, uint4& c1) {
  if constexpr (QM == 1) {
    c0 = make_uint4(pair_byte(x[0], x[1], jb) ^ 0x64806480u, pair_byte(x[2], x[3], jb) ^ 0x64806480u,
                    pair_byte(x[4], x[5], jb) ^ 0x64806480u, pair_byte(x[6], x[7], jb) ^ 0x64806480u);
    c1 = make_uint4(pair_byte(x[0], x[1], jb + 1) ^ 0x64806480u, pair_byte(x[2], x[3], jb + 1) ^ 0x64806480u,
                    pair_byte(x[4], x[5], jb + 1) ^ 0x64806480u, pair_byte(x[6], x[7], jb + 1) ^ 0x64806480u);
  } else {
    // [a.jb, b.jb, a.jb+1, b.jb+1]: the low pair is column jb, the high pair jb + 1
    const uint32_t sel = (uint32_t)jb | ((uint32_t)(4 + jb) << 8) | ((uint32_t)(jb + 1) << 16) |
                         ((uint32_t)(5 + jb) << 24);
    const uint32_t t01 = __builtin_amdgcn_perm(x[1], x[0], sel), t23 = __builtin_amdgcn_perm(x[3], x[2], sel);
    const uint32_t t45 = __builtin_amdgcn_perm(x[5], x[4], sel), t67 = __builtin_amdgcn_perm(x[7], x[6], sel);
    c0 = make_uint4(fp8x2_to_f16x2<false>(t01), fp8x2_to_f16x2<false>(t23), fp8x2_to_f16x2<false>(t45),
                    fp8x2_to_f16x2<false>(t67));
    c1 = make_uint4(fp8x2_to_f16x2<true>(t01), fp8x2_to_f16x2<true>(t23), fp8x2_to_f16x2<true>(t45),
                    fp8x2_to_f16x2<true>(t67));
  }
}

// Two floats as an fp16 pair hi (round to nearest even) plus the fp16 pair of
// the remainders lo (~22 significant bits together).
__device__ __forceinline__ void split_f16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_f16x2(a, b);
  const f16x2v_t h = __builtin_bit_cast(f16x2v_t, hi);
  lo = pack_f16x2(a - (float)h.x, b - (float)h.y);
}
__device__ __forceinline__ float f16x2_sum(uint32_t w) {
  const f16x2v_t h = __builtin_bit_cast(f16x2v_t, w);
  return (float)h.x + (float)h.y;
}

template <int HS>
struct Geo {
  static constexpr int NK = HS / 32;            // QK k-steps; code words per lane per half tile
  static constexpr int NS = HS / 16;            // PV n-steps
  static constexpr int RDW = HS / 128;          // V column regions: 32-bit words (8 columns / lane)
  static constexpr int RUS = (HS % 128) / 64;   //                   16-bit words (4 columns / lane)
  static constexpr int RBY = (HS % 64) / 32;    //                   bytes        (2 columns / lane)
  static constexpr int NVR = RDW + RUS + RBY;   // V words per token per lane
};

// V region r of head size HS: columns per lane (w), first column (cb).
template <int HS>
__device__ __forceinline__ void v_region(int r, int& w, int& cb) {
  constexpr int RDW = Geo<HS>::RDW, RUS = Geo<HS>::RUS;
  if (r < RDW) { w = 8; cb = 128 * r; }
  else if (r < RDW + RUS) { w = 4; cb = 128 * RDW; }
  else { w = 2; cb = 128 * RDW + 64 * RUS; }
}

// ... and of the int8 / fp8 caches: 64-column regions with 4 columns per
// lane (one code word), then a 32-column tail with 2 per lane (head size 96).
template <int HS, int QM>
__device__ __forceinline__ void v_region_any(int r, int& w, int& cb) {
  if constexpr (QM != 0) {
    w = r < HS / 64 ? 4 : 2;
    cb = 64 * r;
  } else {
    v_region<HS>(r, w, cb);
  }
}

template <int HS>
__device__ __forceinline__ void load_k_words(const uint8_t* p, uint32_t (&w)[Geo<HS>::NK]) {
  constexpr int NK = Geo<HS>::NK;
  if constexpr (NK == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x; w[1] = x.y;
  } else if constexpr (NK == 3) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    w[0] = q[0]; w[1] = q[1]; w[2] = q[2];
  } else if constexpr (NK == 4) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (NK == 8) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    const uint4 y = *reinterpret_cast<const uint4*>(p + 16);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    w[4] = y.x; w[5] = y.y; w[6] = y.z; w[7] = y.w;
  } else {
#pragma unroll
    for (int i = 0; i < NK; i += 2) {
      const uint2 x = *reinterpret_cast<const uint2*>(p + 4 * i);
      w[i] = x.x; w[i + 1] = x.y;
    }
  }
}

// The code word(s) of V column chunk m of one token row.
template <int HS>
__device__ __forceinline__ void load_v_words(const uint8_t* row, int m, uint32_t (&w)[Geo<HS>::NVR]) {
  constexpr int RDW = Geo<HS>::RDW, RUS = Geo<HS>::RUS, RBY = Geo<HS>::RBY;
#pragma unroll
  for (int r = 0; r < RDW; ++r) w[r] = *reinterpret_cast<const uint32_t*>(row + 64 * r + 4 * m);
  if constexpr (RUS) w[RDW] = *reinterpret_cast<const uint16_t*>(row + 64 * RDW + 2 * m);
  if constexpr (RBY) w[RDW + RUS] = row[64 * RDW + 32 * RUS + m];
}

struct Unit {
  int s, i0, qbeg, qlen, L, g, ht, sp;
};

// Dense unit index -> (sequence, tile, head tile, kv head group, split);
// called by all lanes of a wave with a wave-uniform u. prefix[s] is the first
// unit of sequence s; unit order inside a sequence is kv head group (plan.hpw
// consecutive kv heads) fastest, then head tile, then split, then query tile.
__device__ __forceinline__ bool decode_unit(const AttnArgs& a, const int32_t* prefix, int u, Unit& un) {
  const int s = wave_search_le(prefix, a.num_seqs, u);
  int64_t qb, qe, L;
  seq_extent(a, s, qb, qe, L);
  const int split = a.plan.split_tokens;
  int nsp = (int)((L + split - 1) / split);
  nsp = nsp < 1 ? 1 : (nsp > a.plan.num_splits ? a.plan.num_splits : nsp);
  const int n_hg = a.nkv / a.plan.hpw;
  int v = u - prefix[s];
  un.g = v % n_hg;
  v /= n_hg;
  un.ht = v % a.plan.n_head_tiles;
  v /= a.plan.n_head_tiles;
  un.sp = v % nsp;
  const int tile = v / nsp;
  un.s = s;
  un.qbeg = (int)qb;
  un.qlen = (int)(qe - qb);
  un.i0 = tile * a.plan.tq;
  un.L = (int)L;
  return un.i0 < un.qlen;
}

// Work units per sequence and their exclusive prefix (one workgroup); in
// stream-K decode, the 32-token KV steps per sequence instead.
// First 32-token KV step of a one-tile query block (qlen rows at positions
// L - qlen .. L - 1) under a sliding window: its first row sees keys from
// L - qlen - window + 1 on.
__device__ __forceinline__ int sk_first_step(int window, int64_t L, int64_t qlen) {
  const int64_t k = L - qlen - window + 1;
  return (window > 0 && k > 0) ? (int)(k >> 5) : 0;
}

// Work units (stream-K: KV steps, from the 32-token step holding the window
// start) of sequence s.
__device__ __forceinline__ int seq_units(const AttnArgs& a, int s) {
  int64_t qb, qe, L;
  seq_extent(a, s, qb, qe, L);
  if (!served_seq(a, qb, qe)) return 0;   // the prefill kernel's, or another launch's
  if (a.plan.sk) return (qe > qb && L > 0) ? (int)((L + 31) / 32) - sk_first_step(a.window, L, qe - qb) : 0;
  const int split = a.plan.split_tokens;
  int nsp = (int)((L + split - 1) / split);
  nsp = nsp < 1 ? 1 : (nsp > a.plan.num_splits ? a.plan.num_splits : nsp);
  const int ntile = (int)((qe - qb + a.plan.tq - 1) / a.plan.tq);
  return ntile * nsp * a.plan.n_head_tiles * (a.nkv / a.plan.hpw);
}

// Exclusive prefix of seq_units over the sequences, by the NT threads of one
// workgroup: into lds[0 .. num_seqs] (lds[num_seqs] = total; NT / 64 more
// ints of lds hold the wave totals) and, when gout is set, into gout too.
template <int NT>
__device__ void block_prefix(const AttnArgs& a, int32_t* lds, int32_t* gout) {
  constexpr int NW = NT / 64;
  int32_t* wave_tot = lds + a.num_seqs + 1;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry = 0;                                  // the same in every thread
  for (int c0 = 0; c0 < a.num_seqs; c0 += NT) {
    const int s = c0 + tid;
    const int units = s < a.num_seqs ? seq_units(a, s) : 0;
    // inclusive scan inside the wave
    int x = units;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) wave_tot[wv] = x;
    __syncthreads();
    int before = carry, all = carry;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      before += i < wv ? wave_tot[i] : 0;
      all += wave_tot[i];
    }
    if (s < a.num_seqs) {
      lds[s] = before + x - units;
      if (gout) gout[s] = before + x - units;
    }
    carry = all;
    __syncthreads();                              // wave_tot is rewritten next round
  }
  if (tid == 0) {
    lds[a.num_seqs] = carry;
    if (gout) gout[a.num_seqs] = carry;
  }
  __syncthreads();
}

// The prefix as its own one-workgroup kernel (calls whose sequences do not
// fit the attention kernel's LDS).
__global__ __launch_bounds__(1024) void attn_plan_kernel(AttnArgs a, int32_t* prefix) {
  __shared__ int32_t lds[1024 + 1 + 16];
  // chunks of 1024 sequences: prefix of the chunk in LDS, then offset by the
  // running total into the global prefix
  int base = 0;
  const int nseq = a.num_seqs;
  for (int c0 = 0; c0 < nseq || c0 == 0; c0 += 1024) {
    AttnArgs c = a;
    c.num_seqs = nseq - c0 < 1024 ? nseq - c0 : 1024;
    c.qsl = a.qsl + c0;
    c.seq_lens = a.seq_lens + c0;
    block_prefix<1024>(c, lds, nullptr);
    for (int i = threadIdx.x; i < c.num_seqs; i += 1024) prefix[c0 + i] = base + lds[i];
    base += lds[c.num_seqs];
    __syncthreads();
    if (c0 + 1024 >= nseq) break;
  }
  if (threadIdx.x == 0) prefix[nseq] = base;
}

// LDS layout of one 32-token step (per wave), filled by direct global->LDS
// loads. A load of `size` bytes puts lane l's bytes at region + l * stride
// with stride = 4 for 1-, 2- and 4-byte loads (sub-dword data zero-extended),
// 16 for 12- and 16-byte loads.
//   K  half h, load j : token (l & 15) of the half tile, code bytes of chunk
//                       l >> 4, words [j * KSZ/4, (j + 1) * KSZ/4)
//   V  token i, region r: token 4 * (l >> 4) + (i & 3) of half tile i >> 2,
//                       column chunk (l & 15) of region r (one dword slot)
//   S  lane l: k_scale (l < 32) / v_scale (l >= 32) of token (l & 15) of half
//                       tile (l >> 4) & 1
template <int HS>
struct StageGeo {
  static constexpr int NK = HS / 32;
  static constexpr int NKL = NK == 2 ? 2 : (NK == 3 ? 1 : (NK == 4 ? 1 : 2));    // K loads per half
  static constexpr int KSZ = NK == 2 ? 4 : (NK == 4 || NK == 8 ? 16 : 12);       // bytes per load
  static constexpr int KSTR = KSZ == 4 ? 4 : 16;                                  // LDS bytes per lane
  static constexpr int KREG = 64 * KSTR;                                          // one K load region
  static constexpr int KHALF = NKL * KREG;                                        // K bytes per half tile
  static constexpr int VBYTES_TOK = 256 * Geo<HS>::NVR;
  // head size 96: packed token rows of the wave's heads, 2 KB per head
  static constexpr int VREG = HS == 96 ? 2048 : 8 * VBYTES_TOK;
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 2 * KHALF;
  static constexpr int S_OFF = V_OFF + VREG;
  static constexpr int BYTES = S_OFF + 256;
};

// Per-token-head int8 / fp8 caches (one byte per element, token rows of HS
// bytes):
//   K  half h, load j : token (l & 15), bytes [HS/4 (l >> 4) + j KSZ, +KSZ)
//                       of its row (HS/4 bytes per lane in 16- or 12-byte
//                       loads, lane stride 16)
//   V  half h         : the 16 token rows packed (row t at t * HS), filled
//                       by 1 KB loads of 16-byte lanes (byte 16 l + 1024 j
//                       of the half tile; lanes past its end fetch nothing)
template <int HS>
struct StageGeoQ {
  static_assert(HS % 32 == 0, "head size");
  static constexpr int KL = HS / 4;                         // K bytes per lane per half tile
  static constexpr int KSZ = KL % 16 == 0 ? 16 : 12;
  static constexpr int NKL = KL / KSZ;
  static constexpr int KSTR = 16, KREG = 1024;
  static constexpr int KHALF = NKL * KREG;
  static constexpr int VL = (16 * HS + 1023) / 1024;      // V loads per half tile
  static constexpr int VHALF = VL * 1024;
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 2 * KHALF;
  static constexpr int S_OFF = V_OFF + 2 * VHALF;
  static constexpr int BYTES = S_OFF + 256;
};
template <int HS, int QM> struct StageSel { using T = StageGeoQ<HS>; };
template <int HS> struct StageSel<HS, 0> { using T = StageGeo<HS>; };

// Stage slots per wave: with kStages slots the loads of steps it + 1 ..
// it + kStages - 1 run during step it. More slots keep more bytes in flight,
// but two measured best: with the cache read from HBM, a third slot at head
// size 64 took a Llama-3.2-1B decode batch from 47.3 to 49.2 us (a fourth
// 52.3), at head size 96 a Phi-3 batch from 43.0 to 44.8, at 128 a Llama-3-8B
// batch from 393 to 406 (one workgroup per CU instead of two) -- these waves
// are bound by instruction issue, not by the loads in flight, and at head
// size 128 the L2 also evicts 128-byte lines before the wave of the
// neighbouring kv head (which reads the other half of the line) gets to them.
template <int HS, int HPW, int QM>
constexpr int stages_for() { return 2; }

// Per wave: kStages stage slots, each holding HPW per-head stages (one per kv
// head the wave serves); the q' staging buffer and the epilogue buffer
// overlay them.
template <int HS, int HPW, int QM, int NRB>
struct MfmaSmem {
  static constexpr int STAGE_H = StageSel<HS, QM>::T::BYTES;   // one kv head
  static constexpr int STAGE = HPW * STAGE_H;               // one slot
  static constexpr int BUFB = 16 * NRB * HS * 4;            // q' staging / epilogue (fp32 rows)
  static constexpr int NST = stages_for<HS, HPW, QM>();
  static constexpr int MAINB = NST * STAGE > BUFB ? NST * STAGE : BUFB;
  alignas(16) unsigned char main[MAINB];
  float qsum[16 * NRB];
  float qrs[16 * NRB];   // int8 / fp8: power of two that undoes the row scaling of q'
};


// The occupancy each HPW is built for: the LDS of HPW per-head stages per
// wave bounds the waves a CU can hold. WPE is the register target (waves per
// SIMD); head size 192 at one head per wave fits two waves (256 registers),
// not three.
template <int HPW> struct MfmaShape;
template <> struct MfmaShape<1> { static constexpr int WPE = 3; };
template <> struct MfmaShape<2> { static constexpr int WPE = 2; };
template <> struct MfmaShape<4> { static constexpr int WPE = 1; };
template <int HS, int HPW, int QM>
constexpr int mfma_wpb() { return mfma_waves_per_block(HPW, QM, HS); }
template <int HS, int HPW, int QM, int NRB = 1>
constexpr int mfma_wpe() {
  // head size 256: the q' pairs and accumulators of one kv head take the
  // whole register file (one wave per SIMD; its two 8.4 KB stage slots
  // still keep ~67 KB per CU in flight)
  if constexpr (HS >= 256) return 1;
  return HPW == 1 && (NRB > 1 || HS >= 192 || (QM != 0 && HS >= 96)) ? 2 : MfmaShape<HPW>::WPE;
}

// HPW = kv heads per wave. HPW = 1: the 16 MFMA rows (32 with NRB = 2) are
// the query tile of one kv head (tq tokens x gh query heads). HPW > 1 (single-token decode): rows
// r = hl * G + i are query head i of kv head kv0 + hl; each head keeps its own
// QK and PV matrix-core products (rows of the other heads are dropped from S
// and zeroed in P), while the softmax, the page walk and the address work are
// shared by the HPW heads.
//
// QM selects the cache: 0 the int4 RHT cache above; 1 / 2 the per-token-head
// int8 / fp8 e4m3fn caches (one byte per element, no rotation; one kv head
// per wave). For those, K and V codes become fp16 operands exactly (int8 with
// the offset 1152 removed through the sums of q' and of P as for int4), QK
// runs on v_mfma_f32_16x16x32_f16 with q' as an fp16 hi + lo pair, and each
// q' row is first scaled by a power of two that puts its largest element in
// [2^14, 2^15) (fp16 keeps its full precision whatever the query's range);
// the logits take the inverse power back.
//
// PH (head size 128, several heads per wave): V staged per head instead of as
// joint token rows of the wave's heads, for layouts whose heads of a token
// row are not adjacent (about 1 % slower than joint rows where they are).
//
// WIN: built with the sliding-window terms (calls without a window run the
// kernel without them).
//
// NT: the K and V code loads carry the non-temporal cache policy. The host
// asks for it where every 128-byte line a wave loads is loaded by that wave
// alone; built for head size 128 (int4 with two or four adjacent heads per
// wave, int8 / fp8) and 256 (int4: one head's 128-byte rows).
//
// NRB (int4, one kv head per wave): 16-row MFMA blocks per wave. With NRB = 2
// one wave serves 32 query rows (a prefill tile, or a multi-token decode
// block of up to 32 / G tokens); the K and V codes of a step become
// operands once and feed both blocks' products, and each block keeps its own
// softmax state (the v_scale exponent e is shared: it depends on the keys
// only).
template <int HS, int HPW, int QM, bool PH, bool WIN, int NRB, bool NT = false, bool PAD = false>
__global__ __launch_bounds__((64 * mfma_wpb<HS, HPW, QM>()))
__attribute__((amdgpu_waves_per_eu(mfma_wpe<HS, HPW, QM, NRB>()))) void attn_mfma_kernel(AttnArgs a,
                                                                                      const int32_t* prefix) {
  static_assert(NRB == 1 || (HPW == 1 && QM == 0), "two row blocks: int4, one kv head per wave");
  // PAD: head sizes 80 and 112 (block size b = 16) on the instances of 96 and
  // 128 (int4, one kv head per wave). The 16 missing columns are zero in q',
  // so whatever K bytes sit there add nothing to the logits, and their output
  // columns are neither written nor merged. Heads start 8-byte aligned (40 and
  // 56 bytes apart), and every code load stays inside the head's hs / 2 bytes:
  // V rows and the K rows of 112 come as 4-byte pieces (a piece past the row's
  // end loads the row's first word again, for a column nothing reads); the K
  // rows of 80 keep their 12-byte pieces, and the last quarter, which would
  // cross the row's end, loads 8 bytes early and its reader takes word 2.
  static_assert(!PAD || (QM == 0 && HPW == 1 && !PH && !NT && (HS == 96 || HS == 128)),
                "padded head sizes: int4, one kv head per wave, 96 / 128 instances");
  using GG = Geo<HS>;
  using SG = typename StageSel<HS, QM>::T;
  using SM = MfmaSmem<HS, HPW, QM, NRB>;
  constexpr int ROWS = 16 * NRB;
  constexpr int WPB = mfma_wpb<HS, HPW, QM>();
  constexpr int NK = GG::NK, NS = GG::NS;
  constexpr int NVR = QM ? (HS + 63) / 64 : GG::NVR;   // V column regions
  constexpr int LP = (HS / 8) <= 8 ? 8 : ((HS / 8) <= 16 ? 16 : 32);   // lanes per row, chunk mapping
  constexpr int RPP = kWave / LP;                                       // rows per pass
  constexpr int HALF = QM ? HS : HS / 2;        // code bytes per token row of one kv head
  static_assert(QM == 0 || HPW == 1, "int8 / fp8: one kv head per wave");
  constexpr int kStages = stages_for<HS, HPW, QM>();
  constexpr int STH = SM::STAGE_H;
  __shared__ SM smem_all[WPB];
  // fused plan: the sequences' prefix, computed by every workgroup
  extern __shared__ int32_t plan_lds[];
  const int32_t* pf = prefix;
  if (a.plan.fused_plan) {
    // the merge reads block 0's copy of the prefix
    block_prefix<64 * WPB>(a, plan_lds, blockIdx.x == 0 ? const_cast<int32_t*>(prefix) : nullptr);
    pf = plan_lds;
  }

  const int lane = threadIdx.x & 63;
  const int wv = WPB == 1 ? 0 : uniform(threadIdx.x >> 6);   // wave index (uniform: LDS bases in SGPRs)
  SM& sm = smem_all[wv];
  float* buf = reinterpret_cast<float*>(sm.main);
  const int n = lane & 15;          // MFMA column: query row of this lane
  const int q4 = lane >> 4;         // 0..3
  const int nkv = a.nkv;
  const int n_hg = nkv / HPW;       // kv head groups
  const int G = a.nq / nkv;
  const int gh = a.plan.gh;
  const int rph = HPW == 1 ? ROWS : a.plan.tq * gh;   // MFMA rows per kv head
  const int split = a.plan.split_tokens;
  const int total = uniform(pf[a.num_seqs]);
  const int bsz = a.bs;
  const int bs_log2 = __builtin_ctz((unsigned)bsz);      // the planner sends only power-of-two pages here
  const int bs_mask = bsz - 1;
  const float inv_b = 1.0f / (float)a.b;
  // One kv head per wave reads half of each 128-byte code line (64-byte rows
  // at head size 128); the neighbouring head's wave reads the other half.
  // With n_hg % WPB == 0 the units of a workgroup are WPB kv heads of one
  // (sequence, query tile, head tile, split): the waves take the same
  // branches and run the same number of steps, and a workgroup barrier per
  // step keeps the two halves of each line together, so each line comes from
  // HBM once. With two or more heads per wave a wave reads whole lines and
  // runs free.
  const bool wg_sync = HPW == 1 && HALF % 128 != 0 && (n_hg % WPB) == 0;

  // lane constants of the chunk mapping (q setup and epilogue)
  const int cj = lane & (LP - 1);
  const bool c_on = cj < HS / 8;
  const int hsv = PAD ? a.hs : HS;                         // the head size of the call (PAD: HS - 16)
  const bool c_live = PAD ? cj < hsv / 8 : c_on;           // a column chunk of the real head
  const uint32_t sbits = (QM == 0 && c_on) ? sign_bits8(a.seed, cj) : 0u;
  uint32_t sx[4];
  sign_xor_bf16x8(sbits, sx);

  // lane byte offsets inside one half tile (relative to its first token row)
  // cache addressing (packed: token rows of nkv * HALF bytes, heads HALF
  // bytes apart; or any layout the caller describes, e.g. scales inline)
  const uint32_t tok_stride = (uint32_t)a.lay.tok;          // bytes between token rows of a page
  const uint32_t head_bytes = (uint32_t)a.lay.head;         // bytes between kv heads of a row
  const uint32_t half_bytes = 16u * tok_stride;             // one half tile of a page
  const int64_t page_bytes = a.lay.blk;                     // one page of one cache
  const int64_t page_rows = a.lay.sblk;                     // scale floats per page
  const int64_t s_tok = a.lay.stok, s_head = a.lay.shead;   // scale floats per token row / head
  constexpr int CA = NT ? 2 : 0;                            // cache policy of the K/V code loads
  const uint32_t koff = (uint32_t)n * tok_stride + (uint32_t)q4 * (HALF / 4) - (PAD && HS == 96 && q4 == 3 ? 8u : 0u);
  // PAD, head size 112: K word w of this lane's quarter (its 4 bytes, or the
  // row's first word past the row's end)
  constexpr bool PADW = PAD && HS == 128;
  uint32_t kw_src[PADW ? 4 : 1];
  if constexpr (PADW) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t b = (uint32_t)q4 * 16u + 4u * (uint32_t)w;
      kw_src[w] = (uint32_t)n * tok_stride + (b < (uint32_t)hsv / 2 ? b : 0u);
    }
  }
  uint32_t vo[4];                                           // token 4*q4 + i, 32-bit column chunk n
#pragma unroll
  for (int i = 0; i < 4; ++i) vo[i] = (uint32_t)(4 * q4 + i) * tok_stride + 4u * (uint32_t)n;
  // Joint V layout (VJ): where the wave's heads make a 64- or 128-byte token
  // row, V comes in with 16-byte lanes and lands token-major in LDS (row
  // after row, RB bytes each, 1 KB per load). Lane l of a load fetches bytes
  // [16 l % RB, +16) of token row 16 l / RB.
  constexpr int RB = HPW * HALF;                            // V bytes per token row of the wave
  // Per-head variant (VJH, head size 128 with several heads per wave): each
  // head's 64-byte rows land in its own stage, so the heads of a token row
  // need not be adjacent in memory.
  constexpr bool VJH = QM == 0 && HPW > 1 && HALF == 64 && PH;
  static_assert(!PH || VJH, "per-head V staging: int4, head size 128, several heads per wave");
  constexpr bool VJ = QM == 0 && !VJH && (RB == 64 || RB == 128);
  constexpr int RPI = 1024 / RB;                            // token rows per 1 KB load (VJ)
  const uint32_t vjh_src = (uint32_t)(lane >> 2) * tok_stride + 16u * (uint32_t)(lane & 3);
  const uint32_t vj_src = (uint32_t)((16 * lane) / RB) * tok_stride + (uint32_t)((16 * lane) % RB);
  // PAD: V as 4-byte pieces, 64 lanes x 4 bytes per load, token-major in LDS
  // (rows of RB bytes) as the 16-byte loads leave them: load k of a half tile
  // takes its dwords 64 k .. 64 k + 63, the row's first word past the row's end
  constexpr int PVL = PAD ? 16 * RB / 256 : 1;            // dword loads per half tile (3 or 4)
  uint32_t pv_src[PVL];
  if constexpr (PAD) {
#pragma unroll
    for (int k = 0; k < PVL; ++k) {
      const int d = 64 * k + lane, t = d / (RB / 4), c = d % (RB / 4);
      pv_src[k] = (uint32_t)t * tok_stride + (4 * c < hsv / 2 ? 4u * (uint32_t)c : 0u);
    }
  }
  // ... and lane (n, q4) reads, for token 4 q4 + i of a half tile, its column
  // chunk n of head hl at vj_rd[i] + hl * HALF: 4 bytes (8 columns, head
  // size 128; int8 / fp8: 4 columns of each 64-column region) or 2 bytes (4
  // columns, head size 64); each 16-lane quarter reads 64 (32) contiguous
  // bytes of one row, so no two of its lanes share an LDS bank.
  // int8 / fp8 (packed token rows, any head size): the source of lane l in V
  // load j of a half tile, and the LDS read offset of lane (n, q4) for token
  // 4 q4 + i (its word n of the row; the 32-column tail: its 16-bit word n)
  uint32_t vq_src[QM ? StageGeoQ<HS>::VL : 1];
  uint32_t vq_rd[4];
  if constexpr (QM != 0) {
#pragma unroll
    for (int j = 0; j < StageGeoQ<HS>::VL; ++j) {
      const int b = 1024 * j + 16 * lane, t = b / HS;
      vq_src[j] = t < 16 ? (uint32_t)t * tok_stride + (uint32_t)(b % HS) : 0x80000000u;   // past the range: zeros
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) vq_rd[i] = (uint32_t)((4 * q4 + i) * HS) + 4u * (uint32_t)n;
  }
  uint32_t vj_rd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 4 * q4 + i;
    vj_rd[i] = VJH ? (uint32_t)(t * 64) + 4u * (uint32_t)n
                   : (uint32_t)((t / RPI) * 1024 + (t % RPI) * RB) + (HS >= 128 ? 4u : 2u) * (uint32_t)n;
  }
  // Packed joint V rows (VP, int4 head size 96): the wave's RB-byte token rows
  // (48 or 96 bytes, six 16-byte pieces per head pair) land token-major in LDS
  // through 16-byte lanes, VPL loads of 1 KB per half tile (lanes past its 16
  // rows fetch nothing). Lane (n, q4) reads 4 bytes (8 columns) of token
  // 4 q4 + i at offset 4 n of its head's 48 bytes, so PV runs as at head size
  // 128: one region of 8 columns per lane, MFMA rows 12-15 (columns 96-127)
  // carrying nothing that is stored.
  constexpr bool VP = QM == 0 && !VJH && HS == 96;
  constexpr int VPL = (16 * RB + 1023) / 1024;
  uint32_t vp_src[VP ? VPL : 1];
  uint32_t vp_rd[4];
  if constexpr (VP) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int b = 1024 * j + 16 * lane, t = b / RB;
      vp_src[j] = t < 16 ? (uint32_t)t * tok_stride + (uint32_t)(b % RB) : 0x80000000u;   // past the range: zeros
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) vp_rd[i] = (uint32_t)((4 * q4 + i) * RB) + 4u * (uint32_t)n;
  }
  // PV column regions (VP: one region of 8 columns per lane) and the V
  // accumulators they need
  constexpr int NVRV = VP ? 1 : NVR;
  constexpr int NSV = VP ? 8 : NS;
  auto vreg = [&](int r, int& w, int& cb) {
    if constexpr (VP) {
      w = 8;
      cb = 0;
    } else {
      v_region_any<HS, QM>(r, w, cb);
    }
  };
  const int64_t soff = (int64_t)(lane & 15) * s_tok;         // scale floats
  const float* sc_base = lane < 32 ? a.k_scale : a.v_scale;
  const bool sc_half_b = (lane & 16) != 0;

  // this lane's MFMA row n: kv head (within the group) and place in the tile
  const int hl_n = n / rph;
  const int rr_n = n - hl_n * rph;
  const int ti_n = rr_n / gh, hi_n = rr_n - (rr_n / gh) * gh;
  const uint32_t hoff_n = (uint32_t)(hl_n < HPW ? hl_n : 0) * STH;   // its head's per-head stage

  // One work unit: the query tile starting at query ui0 of sequence us, kv
  // head group ug, head tile uht, keys [k0, k1). With `partial` the
  // unnormalized result goes to workspace row ptok (split-KV, or stream-K
  // piece) for the merge; otherwise the output is written directly.
  auto run_unit = [&](const int us, const int ui0, const int uqbeg, const int uqlen, const int uL, const int ug,
                      const int uht, const int k0, const int k1, const int64_t ptok0, const bool partial) {
    const int kv0 = ug * HPW;                      // first kv head of this unit
    const int hq0 = uht * gh;                      // first query head of the tile within a group
    const int nh = min(gh, G - hq0);
    const int ntok = min(a.plan.tq, uqlen - ui0);
    const int pos0 = uL - uqlen + ui0;
    // sliding window: row r sees keys (rpos - win, rpos]; a step starting at
    // or after wlo lies in the window of every row of the tile
    const int win = WIN ? a.window : INT_MAX;
    const int wlo = WIN ? pos0 + ntok - a.window : INT_MIN;

    // page ids of this unit, one per lane, 64 pages at a time (loaded first:
    // the q' setup below hides their latency)
    const int32_t* bt = a.block_table + (int64_t)us * a.max_blocks;
    const int npages = k1 > 0 ? ((k1 - 1) >> bs_log2) + 1 : 0;
    int pg0 = k0 >> bs_log2;
    int pg_lane = -1;
    auto load_pages = [&](int first) {
      pg0 = first;
      const int idx = first + lane;
      int p = -1;
      if (idx < npages) {
        p = bt[idx];
        KV4_DBG(p < 0 || p >= a.num_blocks, KV4_DEBUG_PAGE);
        p = (p >= 0 && p < a.num_blocks) ? p : -1;
      }
      pg_lane = p;
    };
    const int nsteps = k1 > k0 ? (k1 - k0 + 31) / 32 : 0;
    if (nsteps > 0) load_pages(pg0);

    // ---- q' rows -> LDS (bf16 hi / lo, k-permuted) and their sums
#pragma unroll
    for (int ps = 0; ps < ROWS / RPP; ++ps) {
      const int r = ps * RPP + lane / LP;
      const int hl = r / rph, rr = r - (r / rph) * rph;
      const int ti = rr / gh, hi = rr - (rr / gh) * gh;
      const bool rv = hl < HPW && ti < ntok && hi < nh;
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (rv && c_live)
        w = *reinterpret_cast<const uint4*>(a.query + (int64_t)(uqbeg + ui0 + ti) * a.q_stride +
                                           (int64_t)((kv0 + hl) * G + hq0 + hi) * hsv + 8 * cj);
      const uint32_t wd[4] = {w.x ^ sx[0], w.y ^ sx[1], w.z ^ sx[2], w.w ^ sx[3]};
      float v[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = bf16_lo(wd[k]);
        v[2 * k + 1] = bf16_hi(wd[k]);
      }
      float sum = 0.0f;
      uint32_t hw[4], lw[4];
      if constexpr (QM == 0) {
        fwht_b_ct<LP>(v, a.b, cj);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // k-order of element offsets [0, 4, 1, 5, 2, 6, 3, 7]
          split_bf16x2(v[k] * a.scale_log2, v[k + 4] * a.scale_log2, hw[k], lw[k]);
          sum += (__uint_as_float(hw[k] << 16) + __uint_as_float(lw[k] << 16)) +
                 (__uint_as_float(hw[k] & 0xFFFF0000u) + __uint_as_float(lw[k] & 0xFFFF0000u));
        }
      } else {
        float mx = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[e] *= a.scale_log2;
          mx = fmaxf(mx, fabsf(v[e]));
        }
#pragma unroll
        for (int d = 1; d < LP; d <<= 1) mx = fmaxf(mx, xor_lane_rt(mx, d));
        // 2^sh puts the row maximum in [2^14, 2^15); sh is kept where both
        // 2^sh and 2^-sh are normal floats
        int sh = 141 - (int)((__float_as_uint(mx) >> 23) & 0xFFu);
        sh = sh < -126 ? -126 : (sh > 126 ? 126 : sh);
        const float f = __uint_as_float((uint32_t)(sh + 127) << 23);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // natural element order
          split_f16x2(v[2 * k] * f, v[2 * k + 1] * f, hw[k], lw[k]);
          sum += f16x2_sum(hw[k]) + f16x2_sum(lw[k]);
        }
        if (cj == 0) sm.qrs[r] = __uint_as_float((uint32_t)(127 - sh) << 23);
      }
      sum = group_sum_ct<LP>(c_on ? sum : 0.0f);
      if (c_on) {
        reinterpret_cast<uint4*>(buf)[(r * HS + 8 * cj) / 8] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        reinterpret_cast<uint4*>(buf)[(ROWS * HS + r * HS + 8 * cj) / 8] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
      if (cj == 0) sm.qsum[r] = sum;
    }
    __builtin_amdgcn_wave_barrier();
    uint4 qh[NRB][NK], ql[NRB][NK];
    float qbias[NRB], qrs_n[NRB], row_add[NRB];
    bool row_ok[NRB];
    int rpos[NRB], ti_b[NRB], hi_b[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int rn = 16 * rb + n;                      // this lane's row in block rb
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        qh[rb][s] = reinterpret_cast<const uint4*>(buf)[(rn * HS + q4 * (HS / 4) + 8 * s) / 8];
        ql[rb][s] = reinterpret_cast<const uint4*>(buf)[(ROWS * HS + rn * HS + q4 * (HS / 4) + 8 * s) / 8];
      }
      // sum of q' times the operand offset of the K codes (int4 136, int8 1152)
      qbias[rb] = (QM == 0 ? 136.0f : (QM == 1 ? 1152.0f : 0.0f)) * sm.qsum[rn];
      qrs_n[rb] = QM == 0 ? 1.0f : sm.qrs[rn];
      const int hl = NRB == 1 ? hl_n : 0;
      const int rr = NRB == 1 ? rr_n : rn;
      ti_b[rb] = NRB == 1 ? ti_n : rr / gh;
      hi_b[rb] = NRB == 1 ? hi_n : rr - (rr / gh) * gh;
      row_ok[rb] = hl < HPW && ti_b[rb] < ntok && hi_b[rb] < nh;
      rpos[rb] = row_ok[rb] ? pos0 + ti_b[rb] : -1;
      row_add[rb] = row_ok[rb] ? 0.0f : -INFINITY;     // invalid rows never get weight
    }
    // the staged q' has been read into registers before the stages overwrite it
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();

    f32x4_t acc[NRB][NSV];
    f32x4_t pacc[NRB];
    float m_run[NRB], l_run[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
      for (int i = 0; i < NSV; ++i) acc[rb][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      pacc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m_run[rb] = -INFINITY;
      l_run[rb] = 0.0f;
    }
    float e_run = -100.0f;   // running v_scale exponent (see the softmax step)

    int okmask = 0;   // bit 2*slot: half A page valid, bit 2*slot+1: half B (wave-uniform)

    // Loads of step `it` into stage slot `it % kStages`, in two groups: K
    // codes + both scales (issue_k, which also looks the pages up), then V
    // codes (issue_v, from the bases issue_k left). Steps past the end issue
    // loads with an empty buffer range (they fetch nothing and fill the slot
    // with zeros, which is never read).
    constexpr int NLK = HPW * (2 * (PADW ? 4 : SG::NKL) + 1);   // loads per issue_k
    constexpr int NLV = PAD ? 2 * PVL
                            : QM ? 2 * StageGeoQ<HS>::VL
                            : (VJH ? 2 * HPW : (VJ ? 2 * (16 / RPI) : (VP ? 2 * VPL : HPW * 8 * NVR)));   // loads per issue_v
    // VJ: half tile hh of a slot (16 * RB bytes) sits in head hh's V region
    // (2 KB; RB = 128 of two heads per wave), at V_OFF + 2 hh KB (RB = 128 of
    // one head, head size 256: its 4 KB V region) or at V_OFF + hh KB (RB = 64)
    auto vj_base = [&](auto* st, int hh) {
      return st + (RB == 128 ? (HPW > 1 ? hh * STH : hh * 2048) : hh * 1024) + SG::V_OFF;
    };
    static_assert(!(VJ && RB == 128 && HPW == 1) || StageGeo<HS>::VREG >= 4096, "one head's V region holds both half tiles");
    // VP: half tile hh in head hh's V region (two heads) or at V_OFF + hh KB (one)
    auto vp_base = [&](auto* st, int hh) { return st + (HPW == 1 ? hh * 1024 : hh * STH) + SG::V_OFF; };
    int64_t v_bya = 0, v_byb = 0;
    uint32_t v_nrec = 0;
    auto issue_k = [&](unsigned char* __restrict__ st, int it) {
      const int slot = it % kStages;
      const bool dummy = it >= nsteps;
      const int base = k0 + 32 * (it < nsteps ? it : 0);
      const int b_in = base + 16 < k1;
      const int pga = base >> bs_log2;
      const int pgb = b_in ? (base + 16) >> bs_log2 : pga;
      int ia = pga - pg0;
      int ib = pgb - pg0;
      if (ia < 0 || ib >= 64) {             // another chunk of the page table (rare)
        wait_vm<0>();
        load_pages(pga);
        ia = 0;
        ib = pgb - pg0;
      }
      int pa = __builtin_amdgcn_readlane(pg_lane, ia);
      int pb = __builtin_amdgcn_readlane(pg_lane, ib);
      const int oka = pa >= 0, okb = pb >= 0 && b_in;
      okmask = (okmask & ~(3 << (2 * slot))) | ((oka | (okb << 1)) << (2 * slot));
      pa = pa < 0 ? 0 : pa;
      pb = pb < 0 ? 0 : pb;
      const int offa = base & bs_mask;
      const int offb = b_in ? (base + 16) & bs_mask : offa;
      // byte offset of the first token row of each half tile inside a cache,
      // and the scale index of that row (first kv head of the unit); head hl
      // of the unit sits hl head strides further on
      const int64_t bya = (int64_t)pa * page_bytes + (int64_t)offa * tok_stride + (int64_t)kv0 * head_bytes;
      const int64_t byb = (int64_t)pb * page_bytes + (int64_t)offb * tok_stride + (int64_t)kv0 * head_bytes;
      int64_t rowa = (int64_t)pa * page_rows + offa * s_tok + kv0 * s_head;
      int64_t rowb = (int64_t)pb * page_rows + offb * s_tok + kv0 * s_head;
      const uint32_t nrec = dummy ? 0u : half_bytes;
      if (dummy) { rowa = 0; rowb = 0; }   // scale rows 0..15 of page 0: lines every wave keeps hot
      v_bya = bya;
      v_byb = byb;
      v_nrec = nrec;
      const __amdgpu_buffer_rsrc_t rk[2] = {rsrc(a.key_cache + bya, nrec),
                                            rsrc(a.key_cache + byb, nrec)};
      const float* scp = sc_base + (sc_half_b ? rowb : rowa) + soff;
#pragma unroll
      for (int hl = 0; hl < HPW; ++hl) {
        unsigned char* sth = st + hl * STH;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if constexpr (PADW) {
            // K word w of every lane at K_OFF + h KHALF + 256 w (KHALF = 1 KB)
#pragma unroll
            for (int w = 0; w < 4; ++w) dma_buf<4, CA>(rk[h], kw_src[w], sth + SG::K_OFF + h * SG::KHALF + w * 256);
          } else {
#pragma unroll
            for (int j = 0; j < SG::NKL; ++j) {
              unsigned char* dst = sth + SG::K_OFF + h * SG::KHALF + j * SG::KREG;
              const uint32_t o = koff + j * SG::KSZ + hl * head_bytes;
              if constexpr (SG::KSZ == 16) dma_buf<16, CA>(rk[h], o, dst);
              else if constexpr (SG::KSZ == 12) dma_buf<12, CA>(rk[h], o, dst);
              else dma_buf<4, CA>(rk[h], o, dst);
            }
          }
        }
        dma(scp + hl * s_head, sth + SG::S_OFF, 4);
      }
    };
    auto issue_v = [&](unsigned char* __restrict__ st) {
      const __amdgpu_buffer_rsrc_t rv[2] = {rsrc(a.value_cache + v_bya, v_nrec),
                                            rsrc(a.value_cache + v_byb, v_nrec)};
      if constexpr (PAD) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int k = 0; k < PVL; ++k)
            dma_buf<4, CA>(rv[hh], pv_src[k], (VP ? vp_base(st, hh) : vj_base(st, hh)) + k * 256);
      } else if constexpr (QM != 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int j = 0; j < StageGeoQ<HS>::VL; ++j)
            dma_buf<16, CA>(rv[hh], vq_src[j], st + SG::V_OFF + hh * StageGeoQ<HS>::VHALF + j * 1024);
      } else if constexpr (VJH) {
#pragma unroll
        for (int hl = 0; hl < HPW; ++hl)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            dma_buf<16, CA>(rv[hh], vjh_src + hl * head_bytes, st + hl * STH + SG::V_OFF + hh * 1024);
      } else if constexpr (VP) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int j = 0; j < VPL; ++j) dma_buf<16, CA>(rv[hh], vp_src[j], vp_base(st, hh) + j * 1024);
      } else if constexpr (VJ) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int j = 0; j < 16 / RPI; ++j)
            dma_buf<16, CA>(rv[hh], vj_src + (uint32_t)(j * RPI) * tok_stride, vj_base(st, hh) + j * 1024);
      } else {
#pragma unroll
        for (int hl = 0; hl < HPW; ++hl) {
          unsigned char* sth = st + hl * STH;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            unsigned char* dst = sth + SG::V_OFF + i * SG::VBYTES_TOK;
            const uint32_t o = vo[i & 3] + hl * head_bytes;
#pragma unroll
            for (int r = 0; r < GG::RDW; ++r) dma_buf<4, CA>(rv[i >> 2], o + 64 * r, dst + r * 256);
            if constexpr (GG::RUS) dma_buf<2, CA>(rv[i >> 2], o - 2u * n + 64 * GG::RDW, dst + GG::RDW * 256);
            if constexpr (GG::RBY)
              dma_buf<1, CA>(rv[i >> 2], o - 3u * n + 64 * GG::RDW + 32 * GG::RUS,
                         dst + (GG::RDW + GG::RUS) * 256);
          }
        }
      }
    };

    if (wg_sync) __builtin_amdgcn_s_barrier();
    // LA = kStages - 1 steps of lookahead: the loads of steps it + 1 ..
    // it + LA fly while step it is computed
    constexpr int LA = kStages - 1;
    constexpr int NLS = NLK + NLV;            // loads per step
    static_assert(LA >= 1 && LA * NLS < 64, "vmcnt range");
    if (nsteps > 0) {
#pragma unroll
      for (int j = 0; j < LA; ++j) {
        issue_k(sm.main + j * SM::STAGE, j);
        issue_v(sm.main + j * SM::STAGE);
      }
    }
    // `st` (read) and `wr` (filled for step it + LA) are distinct slots; the
    // restrict qualifiers let the compiler keep the lookahead loads in flight
    // across the reads of the current step. Outstanding loads at the start of
    // step it, oldest first: K(it), V(it), then K and V of each later step up
    // to it + LA - 1.
    auto step = [&](const unsigned char* __restrict__ st, unsigned char* __restrict__ wr, int it) {
      const int slot = it % kStages;
      const int base = k0 + 32 * it;
      wait_vm<NLV + (LA - 1) * NLS>();        // K and scales of step it landed; V(it) may be in flight
      if (wg_sync) __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue_k(wr, it + LA);                   // into the slot step it - 1 used
      const bool oka = (okmask >> (2 * slot)) & 1, okb = (okmask >> (2 * slot + 1)) & 1;

      // S^T = K . Q'^T per kv head, both half tiles (q' as hi + lo); lane n
      // keeps the logits of its own row's head
      float s8[NRB][8];
      if constexpr (QM != 0) {
        // K codes of this lane: token n, bytes [HS/4 q4, +HS/4), both half tiles
        uint32_t kw[2][2 * NK];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const unsigned char* kr = st + SG::K_OFF + h * SG::KHALF;
#pragma unroll
          for (int j = 0; j < SG::NKL; ++j) {
            const uint32_t* x = reinterpret_cast<const uint32_t*>(kr + j * SG::KREG + 16 * lane);
#pragma unroll
            for (int e = 0; e < SG::KSZ / 4; ++e) kw[h][j * (SG::KSZ / 4) + e] = x[e];
          }
        }
        f32x4_t sa = f32x4_t{0.f, 0.f, 0.f, 0.f}, sb = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NK; ++s) {
          const uint4 ka = k_operand_q<QM>(kw[0][2 * s], kw[0][2 * s + 1]);
          const uint4 kb = k_operand_q<QM>(kw[1][2 * s], kw[1][2 * s + 1]);
          sa = mfma_f16(ka, qh[0][s], sa);
          sb = mfma_f16(kb, qh[0][s], sb);
          sa = mfma_f16(ka, ql[0][s], sa);
          sb = mfma_f16(kb, ql[0][s], sb);
          __builtin_amdgcn_sched_barrier(0);
        }
        s8[0][0] = sa[0]; s8[0][1] = sa[1]; s8[0][2] = sa[2]; s8[0][3] = sa[3];
        s8[0][4] = sb[0]; s8[0][5] = sb[1]; s8[0][6] = sb[2]; s8[0][7] = sb[3];
      } else
#pragma unroll
      for (int hl = 0; hl < HPW; ++hl) {
        // K code words of this lane: token n, chunk q4, both half tiles
        uint32_t kw[2][NK];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const unsigned char* kr = st + hl * STH + SG::K_OFF + h * SG::KHALF;
          if constexpr (PADW) {
#pragma unroll
            for (int w = 0; w < 4; ++w) kw[h][w] = reinterpret_cast<const uint32_t*>(kr + w * 256)[lane];
          } else if constexpr (NK == 4) {
            const uint4 x = *reinterpret_cast<const uint4*>(kr + 16 * lane);
            kw[h][0] = x.x; kw[h][1] = x.y; kw[h][2] = x.z; kw[h][3] = x.w;
          } else if constexpr (NK == 8) {
            // head size 256: two 16-byte loads per half tile (words 4 j .. 4 j + 3)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const uint4 x = *reinterpret_cast<const uint4*>(kr + j * SG::KREG + 16 * lane);
              kw[h][4 * j] = x.x; kw[h][4 * j + 1] = x.y; kw[h][4 * j + 2] = x.z; kw[h][4 * j + 3] = x.w;
            }
          } else if constexpr (NK == 3 || NK == 6) {
#pragma unroll
            for (int j = 0; j < NK / 3; ++j) {
              const uint32_t* x = reinterpret_cast<const uint32_t*>(kr + j * SG::KREG + 16 * lane);
              kw[h][3 * j] = x[0]; kw[h][3 * j + 1] = x[1]; kw[h][3 * j + 2] = x[2];
            }
          } else {
#pragma unroll
            for (int j = 0; j < NK; ++j) kw[h][j] = reinterpret_cast<const uint32_t*>(kr + j * 256)[lane];
          }
        }
        if constexpr (PAD && HS == 96) {
          // the last quarter's 12 bytes were loaded 8 bytes early: its real
          // k-step (0) is word 2
#pragma unroll
          for (int h = 0; h < 2; ++h) kw[h][0] = q4 == 3 ? kw[h][2] : kw[h][0];
        }
        f32x4_t sa[NRB], sb[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          sa[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          sb[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int s = 0; s < NK; ++s) {
          const uint4 ka = k_operand(kw[0][s]), kb = k_operand(kw[1][s]);
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            sa[rb] = mfma_bf16(ka, qh[rb][s], sa[rb]);
            sb[rb] = mfma_bf16(kb, qh[rb][s], sb[rb]);
            sa[rb] = mfma_bf16(ka, ql[rb][s], sa[rb]);
            sb[rb] = mfma_bf16(kb, ql[rb][s], sb[rb]);
          }
          if constexpr (HPW == 1) __builtin_amdgcn_sched_barrier(0);   // one k-step's operands live at a time
        }
        if (hl == 0 || hl == hl_n) {
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            s8[rb][0] = sa[rb][0]; s8[rb][1] = sa[rb][1]; s8[rb][2] = sa[rb][2]; s8[rb][3] = sa[rb][3];
            s8[rb][4] = sb[rb][0]; s8[rb][5] = sb[rb][1]; s8[rb][6] = sb[rb][2]; s8[rb][7] = sb[rb][3];
          }
        }
      }
      const float* scl = reinterpret_cast<const float*>(st + hoff_n + SG::S_OFF);
      const float4 ksa = *reinterpret_cast<const float4*>(&scl[4 * q4]);
      const float4 ksb = *reinterpret_cast<const float4*>(&scl[16 + 4 * q4]);
      const float4 vsa = *reinterpret_cast<const float4*>(&scl[32 + 4 * q4]);
      const float4 vsb = *reinterpret_cast<const float4*>(&scl[48 + 4 * q4]);
      const float ks8[8] = {ksa.x, ksa.y, ksa.z, ksa.w, ksb.x, ksb.y, ksb.z, ksb.w};
      const float vs8[8] = {vsa.x, vsa.y, vsa.z, vsa.w, vsb.x, vsb.y, vsb.z, vsb.w};
      float lg[NRB][8];
      const bool full = base + 32 <= k1 && base + 31 <= pos0 && (!WIN || base >= wlo) && oka && okb;   // wave-uniform
      float mx[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        float dq[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) dq[i] = QM == 0 ? s8[rb][i] - qbias[rb] : (s8[rb][i] - qbias[rb]) * qrs_n[rb];
        if (full) {
#pragma unroll
          for (int i = 0; i < 8; ++i) lg[rb][i] = fmaf(dq[i], ks8[i], row_add[rb]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int tok = base + (i < 4 ? 4 * q4 + i : 16 + 4 * q4 + (i - 4));
            const bool ok =
                tok < k1 && tok <= rpos[rb] && (!WIN || tok > rpos[rb] - win) && (i < 4 ? oka : okb);
            lg[rb][i] = ok ? dq[i] * ks8[i] : -INFINITY;
          }
        }
        mx[rb] = fmaxf(fmaxf(fmaxf(lg[rb][0], lg[rb][1]), fmaxf(lg[rb][2], lg[rb][3])),
                       fmaxf(fmaxf(lg[rb][4], lg[rb][5]), fmaxf(lg[rb][6], lg[rb][7])));
        mx[rb] = max_x16_x32(mx[rb]);
      }
      // p * v_scale enters the matrix cores as one fp16. A power of two 2^-e,
      // e = (exponent of the step's largest v_scale) - 11 kept as a running
      // maximum, holds it below 2^12 and clear of fp16 subnormals; acc, pacc
      // and l all carry the scale 2^-(m + e), m the running logit maximum.
      float vmx = fmaxf(fmaxf(fmaxf(vs8[0], vs8[1]), fmaxf(vs8[2], vs8[3])),
                        fmaxf(fmaxf(vs8[4], vs8[5]), fmaxf(vs8[6], vs8[7])));
      vmx = max_x16_x32(vmx);
      const float e_step = fmaxf((float)((int)((__float_as_uint(vmx) >> 23) & 0xFFu) - 138), -100.0f);
      const float e_new = fmaxf(e_run, e_step);
      uint4 ph4[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float m_new = fmaxf(m_run[rb], mx[rb]);
        const float big_m = (m_new == -INFINITY ? 0.0f : m_new) + e_new;
        // a row that has seen no key yet has nothing to rescale
        const float alpha = m_run[rb] == -INFINITY ? 1.0f : fast_exp2(m_run[rb] + e_run - big_m);
        float psum_l = 0.0f;
        uint32_t pw[4];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const float p0 = fast_exp2(lg[rb][i] - big_m), p1 = fast_exp2(lg[rb][i + 1] - big_m);
          psum_l += p0 + p1;
          pw[i / 2] = pack_f16x2(p0 * vs8[i], p1 * vs8[i + 1]);
        }
        ph4[rb] = make_uint4(pw[0], pw[1], pw[2], pw[3]);
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
          for (int i = 0; i < NSV; ++i) acc[rb][i] *= alpha;
          pacc[rb] *= alpha;
        }
        l_run[rb] = l_run[rb] * alpha + psum_l;
        m_run[rb] = m_new;
      }
      e_run = e_new;

      wait_vm<NLK + (LA - 1) * NLS>();        // V(it) landed; the later steps' loads may be in flight
      __builtin_amdgcn_sched_barrier(0);
      issue_v(wr);

      // O'^T += V^T P^T per kv head, one n-step per V column of this lane's
      // chunks; P^T is zero in the rows of the other heads
      if constexpr (QM != 0) {
        // n-step 4 r + j: column 64 r + 4 m + j in MFMA row m (tail region:
        // 64 r + 2 m + j)
#pragma unroll
        for (int r = 0; r < NVR; ++r) {
          constexpr int R4 = HS / 64;
          uint32_t x[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const unsigned char* src = st + SG::V_OFF + (i >> 2) * StageGeoQ<HS>::VHALF + vq_rd[i & 3];
            if (r < R4) x[i] = *reinterpret_cast<const uint32_t*>(src + 64 * r);
            else x[i] = *reinterpret_cast<const uint16_t*>(src - 2 * n + 64 * R4);
          }
#pragma unroll
          for (int jb = 0; jb < (r < R4 ? 4 : 2); jb += 2) {
            uint4 c0, c1;
            v_operands_q<QM>(x, jb, c0, c1);
            acc[0][4 * r + jb] = mfma_f16(c0, ph4[0], acc[0][4 * r + jb]);
            acc[0][4 * r + jb + 1] = mfma_f16(c1, ph4[0], acc[0][4 * r + jb + 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else
#pragma unroll
      for (int hl = 0; hl < HPW; ++hl) {
        uint4 phh[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) phh[rb] = ph4[rb];
        if constexpr (HPW > 1) {
          const bool mine = hl == hl_n;
          phh[0] = make_uint4(mine ? ph4[0].x : 0u, mine ? ph4[0].y : 0u, mine ? ph4[0].z : 0u, mine ? ph4[0].w : 0u);
        }
        int ns = 0;
#pragma unroll
        for (int r = 0; r < NVRV; ++r) {
          int w, cb;
          vreg(r, w, cb);
          uint32_t x[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if constexpr (VP) {
              x[i] = *reinterpret_cast<const uint32_t*>(vp_base(st, i >> 2) + vp_rd[i & 3] + hl * HALF);
            } else if constexpr (VJH) {
              x[i] = *reinterpret_cast<const uint32_t*>(st + hl * STH + SG::V_OFF + (i >> 2) * 1024 + vj_rd[i & 3]);
            } else if constexpr (VJ) {
              // region r of a 256-wide head: its columns 128 r .. 128 r + 127 are bytes 64 r .. of the row
              const unsigned char* src = vj_base(st, i >> 2) + vj_rd[i & 3] + hl * HALF + 64 * r;
              if constexpr (HS >= 128) x[i] = *reinterpret_cast<const uint32_t*>(src);
              else x[i] = *reinterpret_cast<const uint16_t*>(src);
            } else {
              const unsigned char* src = st + hl * STH + SG::V_OFF + i * SG::VBYTES_TOK;
              // sub-dword regions hold zero-extended words; their unused
              // nibbles are never selected below
              x[i] = reinterpret_cast<const uint32_t*>(src + r * 256)[lane];
            }
          }
#pragma unroll
          for (int jb = 0; jb < 4; ++jb) {
            if (2 * jb >= w) break;
            const uint32_t t01 = pair_byte(x[0], x[1], jb);
            const uint32_t t23 = pair_byte(x[2], x[3], jb);
            const uint32_t t45 = pair_byte(x[4], x[5], jb);
            const uint32_t t67 = pair_byte(x[6], x[7], jb);
            // low nibbles (column 2 jb) moved up to bits 4-7; high nibbles in place
            const uint4 lo = make_uint4(nib2h(t01 << 4), nib2h(t23 << 4), nib2h(t45 << 4), nib2h(t67 << 4));
            const uint4 hi = make_uint4(nib2h(t01), nib2h(t23), nib2h(t45), nib2h(t67));
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
              acc[rb][ns] = mfma_f16(lo, phh[rb], acc[rb][ns]);
              acc[rb][ns + 1] = mfma_f16(hi, phh[rb], acc[rb][ns + 1]);
            }
            ns += 2;
            if constexpr (HPW == 1) __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      if constexpr (QM != 2) {   // fp8 codes carry no offset
        const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);   // fp16 1.0
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) pacc[rb] = mfma_f16(ones, ph4[rb], pacc[rb]);
      }
    };
    for (int it = 0, rs = 0; it < nsteps; ++it) {
      const int ws = rs == 0 ? kStages - 1 : rs - 1;   // slot of step it + LA
      step(sm.main + rs * SM::STAGE, sm.main + ws * SM::STAGE, it);
      rs = rs + 1 == kStages ? 0 : rs + 1;
    }
    wait_vm<0>();                             // no load may land in LDS after this point
    __builtin_amdgcn_wave_barrier();

    // ---- finish: l over the four lane quarters, remove the offset of the
    // fp16 V operands (int4: 64 + u = 72 + code; int8: 1152 + code)
    float pbias[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      l_run[rb] = sum_x16_x32(l_run[rb]);
      pbias[rb] = (QM == 0 ? 72.0f : (QM == 1 ? 1152.0f : 0.0f)) * pacc[rb][0];
    }
    if (partial) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
      const int qrow = uqbeg + ui0 + ti_b[rb];
      const int h = (kv0 + (NRB == 1 ? hl_n : 0)) * G + hq0 + hi_b[rb];
      if (row_ok[rb]) {
        // split-KV: one row per (split, query token); stream-K: one per piece
        // (stream-K: one row per (piece, query token of the tile, q head))
        const int64_t ptok = a.plan.sk ? ptok0 * a.plan.tq + ti_b[rb] : ptok0 + qrow;
        const int64_t prow = ptok * a.nq + h;
        float* dst = a.ws_o + prow * hsv;
        int ns = 0;
#pragma unroll
        for (int r = 0; r < NVRV; ++r) {
          int w, cb;
          vreg(r, w, cb);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            if ((VP || PAD) && 4 * q4 + rr >= hsv / 8) continue;   // MFMA rows past the head's columns
            float* d = dst + cb + w * (4 * q4 + rr);
            const f32x4_t* A = acc[rb];
            const float pb = pbias[rb];
            if (w == 8) {
              reinterpret_cast<float4*>(d)[0] = make_float4(A[ns][rr] - pb, A[ns + 1][rr] - pb,
                                                            A[ns + 2][rr] - pb, A[ns + 3][rr] - pb);
              reinterpret_cast<float4*>(d)[1] = make_float4(A[ns + 4][rr] - pb, A[ns + 5][rr] - pb,
                                                            A[ns + 6][rr] - pb, A[ns + 7][rr] - pb);
            } else if (w == 4) {
              reinterpret_cast<float4*>(d)[0] = make_float4(A[ns][rr] - pb, A[ns + 1][rr] - pb,
                                                            A[ns + 2][rr] - pb, A[ns + 3][rr] - pb);
            } else {
              reinterpret_cast<float2*>(d)[0] = make_float2(A[ns][rr] - pb, A[ns + 1][rr] - pb);
            }
          }
          ns += w;
        }
        if (q4 == 0) {
          a.ws_ml[2 * prow] = m_run[rb] + e_run;   // the scale exponent of this partial
          a.ws_ml[2 * prow + 1] = l_run[rb];
        }
      }
      }
      return;
    }
    // single split: normalize, stage the rows in LDS, inverse rotation, store
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float inv_l = l_run[rb] > 0.0f ? 1.0f / l_run[rb] : 0.0f;
      int ns = 0;
#pragma unroll
      for (int r = 0; r < NVRV; ++r) {
        int w, cb;
        vreg(r, w, cb);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          if (VP && 4 * q4 + rr >= HS / 8) continue;   // MFMA rows past the head's columns
          const int c0 = cb + w * (4 * q4 + rr);
#pragma unroll
          for (int t = 0; t < 8; ++t)
            if (t < w) buf[(16 * rb + n) * HS + c0 + t] = (acc[rb][ns + t][rr] - pbias[rb]) * inv_l;
        }
        ns += w;
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ps = 0; ps < ROWS / RPP; ++ps) {
      const int r = ps * RPP + lane / LP;
      const int hl = r / rph, rr = r - (r / rph) * rph;
      const int ti = rr / gh, hi = rr - (rr / gh) * gh;
      const bool rv = hl < HPW && ti < ntok && hi < nh;
      float o[8];
      if (c_on) {
        const float4 x0 = reinterpret_cast<const float4*>(buf)[(r * HS + 8 * cj) / 4];
        const float4 x1 = reinterpret_cast<const float4*>(buf)[(r * HS + 8 * cj) / 4 + 1];
        o[0] = x0.x; o[1] = x0.y; o[2] = x0.z; o[3] = x0.w;
        o[4] = x1.x; o[5] = x1.y; o[6] = x1.z; o[7] = x1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.0f;
      }
      if constexpr (QM == 0) {
        fwht_b_ct<LP>(o, a.b, cj);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = apply_sign(o[e] * inv_b, sbits, e);
      }
      if (rv && c_live) {
        uint4 wo;
        wo.x = pack_bf16x2(o[0], o[1]);
        wo.y = pack_bf16x2(o[2], o[3]);
        wo.z = pack_bf16x2(o[4], o[5]);
        wo.w = pack_bf16x2(o[6], o[7]);
        *reinterpret_cast<uint4*>(a.out + ((int64_t)(uqbeg + ui0 + ti) * a.nq + (kv0 + hl) * G + hq0 + hi) * hsv +
                                  8 * cj) = wo;
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  if (a.plan.sk) {
    // Single-token decode, stream-K: the KV steps (32 tokens) of every (kv
    // head group quad, sequence) pair, concatenated quad-major, are cut into
    // P = min(gridDim.x, steps) equal contiguous ranges; block w walks its range and runs one
    // unit per sequence piece, its partial named w + quad * num_seqs + s.
    // prefix[s] holds the first step of sequence s, prefix[num_seqs] the total.
    const int nseq = a.num_seqs;
    const int64_t S = total;
    const int64_t W = (int64_t)a.plan.sk_quads * S;   // quads = n_hg / WPB
    // no more ranges than steps, so none is empty (the merge relies on it)
    const int64_t P = min((int64_t)gridDim.x, W);
    const int64_t w = blockIdx.x;
    if (w >= P) return;
    int64_t x = floor_div_small(w * W, P);
    const int64_t x1 = floor_div_small((w + 1) * W, P);
    while (x < x1) {
      const int q = (int)(x / S);
      const int64_t loc = x - (int64_t)q * S;
      const int s_ = wave_search_le(pf, nseq, loc);
      const int64_t t0 = uniform(pf[s_]), t1 = uniform(pf[s_ + 1]);
      const int64_t end = min(x1 - (int64_t)q * S, t1);
      int64_t qb, qe, L;
      seq_extent(a, s_, qb, qe, L);
      const int uqb = uniform((int)qb), uql = uniform((int)(qe - qb)), uL = uniform((int)L);
      const int fs = WIN ? sk_first_step(a.window, uL, uql) : 0;
      const int k0 = (int)(32 * (loc - t0 + fs));
      const int k1 = (int)min((int64_t)32 * (end - t0 + fs), (int64_t)uL);
      run_unit(s_, 0, uqb, uql, uL, q * WPB + wv, 0, k0, k1, w + (int64_t)q * nseq + s_, true);
      x = (int64_t)q * S + end;
    }
    return;
  }

  // Workgroups are dealt to the 8 XCDs round-robin (block b on XCD b % 8).
  // Unit blocks 2k and 2k + 1 (e.g. kv heads 0-3 and 4-7 of one sequence
  // split, whose scale rows share 128-byte lines) go to blocks b and b + 8,
  // which share an XCD and its L2.
  const int nbk = gridDim.x, bk = blockIdx.x;
  const int pbk = bk < (nbk & ~15) ? ((bk & ~15) | ((bk & 7) << 1) | ((bk >> 3) & 1)) : bk;
  for (int u0 = pbk * WPB; u0 < total; u0 += gridDim.x * WPB) {
    const int u = u0 + wv;
    if (u >= total) continue;
    Unit un;
    if (!decode_unit(a, pf, u, un)) continue;
    // the unit is the same for every lane of the wave
    const int us = uniform(un.s), ui0 = uniform(un.i0), uqbeg = uniform(un.qbeg);
    const int uqlen = uniform(un.qlen), uL = uniform(un.L), ug = uniform(un.g);
    const int uht = uniform(un.ht), usp = uniform(un.sp);
    const int ntok = min(a.plan.tq, uqlen - ui0);
    const int kend = uL - uqlen + ui0 + ntok;
    // keys below the tile's first sliding window start (32-aligned) are not read
    const int kwin = WIN ? (max(0, uL - uqlen + ui0 - a.window + 1) & ~31) : 0;
    const int k0 = max(usp * split, kwin);
    const int k1 = min(usp * split + split, kend);
    if (k0 >= k1 && usp > 0) continue;   // no keys for this tile in this split (the merge skips it)
    // split partial rows: (split, query token) rows, or beside the prefill
    // kernel (sequences of at most q_hi queries here) mostly the compact
    // (split, sequence, query of the sequence) rows
    const int64_t ptok0 = compact_rows(a.plan)
                              ? ((int64_t)usp * a.num_seqs + us) * a.plan.q_hi - uqbeg
                              : (int64_t)usp * a.num_q_tokens;
    run_unit(us, ui0, uqbeg, uqlen, uL, ug, uht, k0, k1, ptok0, a.plan.num_splits > 1);
  }
}

// Attributes of the current device that the launch geometry depends on,
// read once per device (several GPUs of different kinds may be used from one
// process, from several threads).
struct DevAttrs {
  int dev;
  int cus;
  int lds_per_cu;
};

static DevAttrs device_attrs() {
  static std::mutex mu;
  static std::unordered_map<int, DevAttrs> by_dev;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  std::lock_guard<std::mutex> lock(mu);
  auto it = by_dev.find(dev);
  if (it != by_dev.end()) return it->second;
  DevAttrs d{dev, 256, 160 * 1024};
  int v = 0;
  if (dev >= 0 && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
    d.cus = v;
  if (dev >= 0 && hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess &&
      v > 0)
    d.lds_per_cu = v;
  by_dev.emplace(dev, d);
  return d;
}

// Sequences whose prefix the attention kernel computes itself (in LDS) when
// that costs it no occupancy; longer batches run the plan kernel first.
constexpr int kFusedPlanMaxSeqs = 1024;
// LDS of the fused prefix for num_seqs sequences (the prefix, its total and
// one partial sum per wave), in 1 KB steps: small batches reserve little
// LDS and keep the kernel's occupancy.
inline size_t fused_plan_lds(int num_seqs) {
  return ((size_t)(num_seqs + 1 + 16) * sizeof(int32_t) + 1023) / 1024 * 1024;
}

// Whether the plan LDS leaves the kernel's resident workgroups per CU as
// they are, counting LDS in 1 KB units: the occupancy query counts bytes,
// and a kernel whose workgroups fill the CU to within a few hundred bytes
// (head size 192, int8 / fp8: three of 50.4 KB) was measured to lose a
// workgroup per CU with the plan LDS although the query said otherwise.
static bool plan_lds_fits(const void* kernel, int resident, size_t plan_lds, const DevAttrs& da) {
  // static LDS of each kernel, looked up once (the same code object on every device)
  static std::mutex mu;
  static std::unordered_map<const void*, size_t> static_lds;
  size_t lds = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = static_lds.find(kernel);
    if (it == static_lds.end()) {
      hipFuncAttributes fa;
      if (hipFuncGetAttributes(&fa, kernel) != hipSuccess) return false;
      it = static_lds.emplace(kernel, fa.sharedSizeBytes).first;
    }
    lds = it->second;
  }
  const size_t per_wg = (lds + plan_lds + 1023) / 1024 * 1024;
  const int per_cu = resident / (da.cus > 0 ? da.cus : 1);
  return (size_t)per_cu * per_wg <= (size_t)da.lds_per_cu;
}

// Workgroups of the kernel the GPU holds at once (fused: with the plan LDS).
// (per device: the occupancy query is answered for the current device), with
// plan_lds bytes of dynamic LDS (the fused prefix; 0 without it)
template <int HS, int HPW, int QM, bool PH, bool WIN, int NRB = 1, bool NT = false, bool PAD = false>
static int resident_blocks(size_t plan_lds, const DevAttrs& da) {
  static std::mutex mu;
  static std::unordered_map<int64_t, int> per_cu;      // key: device, LDS
  const int64_t key = (int64_t)da.dev * (1 << 20) + (int64_t)plan_lds;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = per_cu.find(key);
    if (it != per_cu.end()) return it->second * da.cus;
  }
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb,
                                                   reinterpret_cast<const void*>(&attn_mfma_kernel<HS, HPW, QM, PH, WIN, NRB, NT, PAD>),
                                                   64 * mfma_wpb<HS, HPW, QM>(), plan_lds) != hipSuccess ||
      nb < 1)
    nb = 1;
  std::lock_guard<std::mutex> lock(mu);
  per_cu.emplace(key, nb);
  return nb * da.cus;
}

template <int HS, int QM, bool WIN>
static hipError_t launch_hs_w(AttnArgs& a, const int32_t* prefix, int64_t max_units, hipStream_t stream) {
  if (a.plan.hpw == 4 && Geo<HS>::NVR != 1) return hipErrorInvalidValue;
  if (QM != 0 && (a.plan.hpw != 1 || a.plan.wpb != mfma_wpb<HS, 1, QM>())) return hipErrorInvalidValue;
  // resident(fused, device) -> workgroups the GPU holds at once
  const DevAttrs da = device_attrs();
  const size_t plan_lds = fused_plan_lds(a.num_seqs);
  auto go = [&](auto kernel, int wpb, auto resident_of) {
    const int plain = resident_of((size_t)0, da);
    // the workgroups the launch wants at once: stream-K at most its cap; the
    // prefix is built in-kernel where its LDS leaves room for that many
    const int want = a.plan.sk ? std::min(plain, a.plan.sk_pcap) : plain;
    const int with_plan = resident_of(plan_lds, da);
    a.plan.fused_plan = (a.num_seqs <= kFusedPlanMaxSeqs && with_plan >= want &&
                         plan_lds_fits(reinterpret_cast<const void*>(kernel), want, plan_lds, da)) ? 1 : 0;
    if (const char* f = std::getenv("KV4_FUSED_PLAN")) a.plan.fused_plan = a.plan.fused_plan && std::atoi(f) != 0;
    if (std::getenv("KV4_DEBUG_PLAN")) {
      hipFuncAttributes fa{};
      (void)hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kernel));
      std::fprintf(stderr,
                   "[kv4] hs %d hpw %d qm %d rb %d sk %d: resident %d (with %zu B prefix LDS: %d), static LDS %zu, "
                   "LDS/CU %d, CUs %d, fused prefix %d\n",
                   HS, a.plan.hpw, QM, a.plan.rb, a.plan.sk, plain, plan_lds, with_plan,
                   (size_t)fa.sharedSizeBytes, da.lds_per_cu, da.cus, a.plan.fused_plan);
    }
    const int resident = a.plan.fused_plan ? std::min(plain, with_plan) : plain;
    if (!a.plan.fused_plan)
      hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(1024), 0, stream, a, const_cast<int32_t*>(prefix));
    int64_t wgs;
    if (a.plan.sk) {
      // stream-K: exactly the workgroups the GPU holds at once (at most the
      // planner's cap, which sized the workspace)
      wgs = std::min<int64_t>(resident, a.plan.sk_pcap);
      if (a.plan.sk_per_cu > 0) wgs = std::min<int64_t>(wgs, (int64_t)da.cus * a.plan.sk_per_cu);
      a.plan.sk_grid = (int)std::max<int64_t>(wgs, 1);
      wgs = a.plan.sk_grid;
    } else {
      wgs = (max_units + wpb - 1) / wpb;
      const int64_t cap = a.plan.wg_cap > 0 ? std::min<int64_t>(a.plan.wg_cap, (int64_t)da.cus * 8) : (int64_t)da.cus * 8;
      if (wgs > cap) wgs = cap;
      if (wgs < 1) wgs = 1;
    }
    hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(64 * wpb), a.plan.fused_plan ? plan_lds : 0, stream, a,
                       prefix);
  };
  if (a.hs != HS) {
    // head sizes 80 / 112 on the 96 / 128 instances (int4, one kv head per wave)
    if constexpr (QM == 0 && (HS == 96 || HS == 128)) {
      if (a.hs != HS - 16 || a.plan.hpw != 1 || a.plan.vjh || a.code_nt) return hipErrorInvalidValue;
      if (a.plan.rb == 2)
        go(attn_mfma_kernel<HS, 1, 0, false, WIN, 2, false, true>, mfma_wpb<HS, 1, 0>(),
           [](size_t l, const DevAttrs& d) { return resident_blocks<HS, 1, 0, false, WIN, 2, false, true>(l, d); });
      else
        go(attn_mfma_kernel<HS, 1, 0, false, WIN, 1, false, true>, mfma_wpb<HS, 1, 0>(),
           [](size_t l, const DevAttrs& d) { return resident_blocks<HS, 1, 0, false, WIN, 1, false, true>(l, d); });
      return hipSuccess;
    }
    return hipErrorInvalidValue;
  }
  if constexpr (QM != 0) {
    if constexpr (HS == 128) {
      if (a.code_nt) {
        go(attn_mfma_kernel<HS, 1, QM, false, WIN, 1, true>, mfma_wpb<HS, 1, QM>(),
           [](size_t l, const DevAttrs& d) { return resident_blocks<HS, 1, QM, false, WIN, 1, true>(l, d); });
        return hipSuccess;
      }
    }
    go(attn_mfma_kernel<HS, 1, QM, false, WIN, 1>, mfma_wpb<HS, 1, QM>(), [](size_t l, const DevAttrs& d) { return resident_blocks<HS, 1, QM, false, WIN>(l, d); });
    return hipSuccess;
  }
  if (a.plan.vjh) {
    if constexpr (HS == 128) {
      if (a.plan.hpw == 2) {
        go(attn_mfma_kernel<HS, 2, 0, true, WIN, 1>, mfma_wpb<HS, 2, 0>(), [](size_t l, const DevAttrs& d) { return resident_blocks<HS, 2, 0, true, WIN>(l, d); });
      } else if (a.plan.hpw == 4) {
        go(attn_mfma_kernel<HS, 4, 0, true, WIN, 1>, mfma_wpb<HS, 4, 0>(), [](size_t l, const DevAttrs& d) { return resident_blocks<HS, 4, 0, true, WIN>(l, d); });
      } else {
        return hipErrorInvalidValue;
      }
      return hipSuccess;
    }
    return hipErrorInvalidValue;
  }
  if (a.plan.rb == 2) {
    if constexpr (HS <= 128) {
      go(attn_mfma_kernel<HS, 1, 0, false, WIN, 2>, mfma_wpb<HS, 1, 0>(), [](size_t l, const DevAttrs& d) { return resident_blocks<HS, 1, 0, false, WIN, 2>(l, d); });
      return hipSuccess;
    }
    return hipErrorInvalidValue;
  }
  if constexpr (HS == 256) {
    if (a.code_nt && a.plan.hpw == 1) {
      go(attn_mfma_kernel<HS, 1, 0, false, WIN, 1, true>, mfma_wpb<HS, 1, 0>(),
         [](size_t l, const DevAttrs& d) { return resident_blocks<HS, 1, 0, false, WIN, 1, true>(l, d); });
      return hipSuccess;
    }
  }
  if constexpr (HS == 128) {
    if (a.code_nt && a.plan.hpw == 2) {
      go(attn_mfma_kernel<HS, 2, 0, false, WIN, 1, true>, mfma_wpb<HS, 2, 0>(),
         [](size_t l, const DevAttrs& d) { return resident_blocks<HS, 2, 0, false, WIN, 1, true>(l, d); });
      return hipSuccess;
    }
    if (a.code_nt && a.plan.hpw == 4) {
      go(attn_mfma_kernel<HS, 4, 0, false, WIN, 1, true>, mfma_wpb<HS, 4, 0>(),
         [](size_t l, const DevAttrs& d) { return resident_blocks<HS, 4, 0, false, WIN, 1, true>(l, d); });
      return hipSuccess;
    }
  }
  switch (a.plan.hpw) {
    case 2: go(attn_mfma_kernel<HS, 2, 0, false, WIN, 1>, mfma_wpb<HS, 2, 0>(), [](size_t l, const DevAttrs& d) { return resident_blocks<HS, 2, 0, false, WIN>(l, d); }); break;
    case 4:
      // four heads' V loads of a step must fit the 6-bit load counter
      if constexpr (Geo<HS>::NVR == 1)
        go(attn_mfma_kernel<HS, 4, 0, false, WIN, 1>, mfma_wpb<HS, 4, 0>(), [](size_t l, const DevAttrs& d) { return resident_blocks<HS, 4, 0, false, WIN>(l, d); });
      break;
    default: go(attn_mfma_kernel<HS, 1, 0, false, WIN, 1>, mfma_wpb<HS, 1, 0>(), [](size_t l, const DevAttrs& d) { return resident_blocks<HS, 1, 0, false, WIN>(l, d); }); break;
  }
  return hipSuccess;
}

template <int HS, int QM>
static hipError_t launch_hs(AttnArgs& a, const int32_t* prefix, int64_t max_units, hipStream_t stream) {
  if (a.window > 0) return launch_hs_w<HS, QM, true>(a, prefix, max_units, stream);
  return launch_hs_w<HS, QM, false>(a, prefix, max_units, stream);
}

hipError_t launch_attn_mfma(AttnArgs& a, int32_t* prefix, int64_t max_units, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (a.qm == 0) {
    switch (a.hs) {
      case 64: e = launch_hs<64, 0>(a, prefix, max_units, stream); break;
      case 80:
      case 96: e = launch_hs<96, 0>(a, prefix, max_units, stream); break;
      case 112:
      case 128: e = launch_hs<128, 0>(a, prefix, max_units, stream); break;
      case 192: e = launch_hs<192, 0>(a, prefix, max_units, stream); break;
      case 256: e = launch_hs<256, 0>(a, prefix, max_units, stream); break;
      default: return hipErrorInvalidValue;
    }
  } else if (a.qm == 1 || a.qm == 2) {
    const bool q1 = a.qm == 1;
    switch (a.hs) {
      case 64: e = q1 ? launch_hs<64, 1>(a, prefix, max_units, stream) : launch_hs<64, 2>(a, prefix, max_units, stream); break;
      case 96: e = q1 ? launch_hs<96, 1>(a, prefix, max_units, stream) : launch_hs<96, 2>(a, prefix, max_units, stream); break;
      case 128:
        e = q1 ? launch_hs<128, 1>(a, prefix, max_units, stream) : launch_hs<128, 2>(a, prefix, max_units, stream);
        break;
      case 192:
        e = q1 ? launch_hs<192, 1>(a, prefix, max_units, stream) : launch_hs<192, 2>(a, prefix, max_units, stream);
        break;
      case 256:
        e = q1 ? launch_hs<256, 1>(a, prefix, max_units, stream) : launch_hs<256, 2>(a, prefix, max_units, stream);
        break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

KV4_DEBUG_ACCESSOR(debug_flags_mfma)

}  // namespace kv4
