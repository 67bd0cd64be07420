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
// rows, kv head, KV split); a workgroup of 4 waves takes 4 consecutive units
// (consecutive kv heads of the same pages when num_kv_heads >= 4, so their
// 16-byte code rows share cache lines inside one CU). The KV range is walked
// 32 tokens (two 16-token half tiles) per step:
//   * S^T = K . Q'^T on v_mfma_f32_16x16x32_bf16: A = K codes (16 tokens x 32
//     head elements), B = q' rows (bf16). The head dimension is permuted so
//     that a lane's 16 / 12 / 8 ... code bytes of one token are one vector
//     load and feed all k-steps; q' is permuted the same way.
//   * q' and p * v_scale enter as bf16 hi + lo pairs (two MFMAs each), so
//     the products carry ~16 significant bits: sharp softmax rows (large
//     k_scale from outlier channels) stay within 1e-2 of the fp64 result.
//   * Codes become bf16 operands exactly, two per VALU op: (u & 0xF) |
//     0x4300 is the bf16 of 128 + u with u = code + 8 (nibble xor 8). The
//     constant 136 is removed after the product with the sum of q' (QK) and
//     with the sum of p*v_scale (PV, obtained from one extra MFMA against a
//     ones operand, so it sees exactly the rounded operands).
//   * The S^T accumulator leaves each lane with 8 logits of ONE query row,
//     which is exactly the B-operand layout P^T needs for O'^T = V^T P^T, so
//     softmax runs in registers with no transpose; the V^T operand is built
//     from 8 tokens' code words per lane (byte permutes + masks).
//   * k_scale / v_scale of the 32 tokens are loaded once per step (one lane
//     per token) and redistributed through a 256-byte LDS slot per wave.
// Pages are looked up once per 16-token half tile (block_size % 16 == 0).
#include "kv4_device.hpp"
#include "kv4_launch.hpp"

namespace kv4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Nibble pair -> bf16 pair: for the nibbles at bits 0-3 and 16-19 of x,
// (nibble ^ 8) | 0x4300, i.e. the bf16 of 128 + u with u = code + 8; every
// other bit comes from the constant. One v_bitop3 (out = m ? x ^ k : k).
__device__ __forceinline__ uint32_t nib2bf(uint32_t x) {
  return __builtin_amdgcn_bitop3_b32(x, 0x43084308u, 0x000F000Fu, 0x6C);
}

// 8 codes of one token (one 32-bit word) -> A operand of one k-step, in
// k-order of element offsets [0, 4, 1, 5, 2, 6, 3, 7].
__device__ __forceinline__ uint4 k_operand(uint32_t w) {
  return make_uint4(nib2bf(w), nib2bf(w >> 4), nib2bf(w >> 8), nib2bf(w >> 12));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats as a bf16 pair hi (round to nearest even, v_cvt_pk_bf16_f32)
// plus the bf16 pair of the remainders lo: hi + lo carries ~16 significant
// bits, which keeps sharp softmax rows (large k_scale) accurate.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
  const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xFFFF0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a - ha, b - hb}, bf16x2_t));
}

// bytes jb of two words -> [a.jb, 0, b.jb, 0]
__device__ __forceinline__ uint32_t pair_byte(uint32_t a, uint32_t b, int jb) {
  const uint32_t sel = (uint32_t)jb | (0x0Cu << 8) | ((uint32_t)(4 + jb) << 16) | (0x0Cu << 24);
  return __builtin_amdgcn_perm(b, a, sel);
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

// Dense unit index -> (sequence, tile, head tile, kv head, split); called by
// all lanes of a wave with a wave-uniform u. prefix[s] is the first unit of
// sequence s; unit order inside a sequence is kv head
// fastest, then head tile, then split, then query tile.
__device__ __forceinline__ bool decode_unit(const AttnArgs& a, const int32_t* prefix, int u, Unit& un) {
  const int s = wave_search_le(prefix, a.num_seqs, u);
  int64_t qb = a.qsl[s], qe = a.qsl[s + 1];
  qb = qb < 0 ? 0 : (qb > a.num_q_tokens ? a.num_q_tokens : qb);
  qe = qe < qb ? qb : (qe > a.num_q_tokens ? a.num_q_tokens : qe);
  int64_t L = a.seq_lens[s];
  const int64_t cap = (int64_t)a.max_blocks * a.bs;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int split = a.plan.split_tokens;
  int nsp = (int)((L + split - 1) / split);
  nsp = nsp < 1 ? 1 : (nsp > a.plan.num_splits ? a.plan.num_splits : nsp);
  int v = u - prefix[s];
  un.g = v % a.nkv;
  v /= a.nkv;
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

// Work units per sequence and their exclusive prefix (one workgroup).
__global__ __launch_bounds__(1024) void attn_plan_kernel(AttnArgs a, int32_t* prefix) {
  __shared__ int32_t wave_tot[16];
  __shared__ int32_t carry;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  const int split = a.plan.split_tokens;
  for (int c0 = 0; c0 < a.num_seqs; c0 += 1024) {
    const int s = c0 + tid;
    int units = 0;
    if (s < a.num_seqs) {
      int64_t qb = a.qsl[s], qe = a.qsl[s + 1];
      qb = qb < 0 ? 0 : (qb > a.num_q_tokens ? a.num_q_tokens : qb);
      qe = qe < qb ? qb : (qe > a.num_q_tokens ? a.num_q_tokens : qe);
      int64_t L = a.seq_lens[s];
      const int64_t cap = (int64_t)a.max_blocks * a.bs;
      L = L < 0 ? 0 : (L > cap ? cap : L);
      int nsp = (int)((L + split - 1) / split);
      nsp = nsp < 1 ? 1 : (nsp > a.plan.num_splits ? a.plan.num_splits : nsp);
      const int ntile = (int)((qe - qb + a.plan.tq - 1) / a.plan.tq);
      units = ntile * nsp * a.plan.n_head_tiles * a.nkv;
    }
    // inclusive scan inside the wave
    int x = units;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) wave_tot[wv] = x;
    __syncthreads();
    int before = carry;
    for (int i = 0; i < wv; ++i) before += wave_tot[i];
    if (s < a.num_seqs) prefix[s] = before + x - units;
    __syncthreads();
    if (tid == 1023) carry = before + x;
    __syncthreads();
  }
  if (tid == 0) prefix[a.num_seqs] = carry;
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
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 2 * KHALF;
  static constexpr int S_OFF = V_OFF + 8 * VBYTES_TOK;
  static constexpr int BYTES = S_OFF + 256;
  static constexpr int LOADS = 2 * NKL + 8 * Geo<HS>::NVR + 1;   // VMEM instructions per step
};

// stage slots per wave: loads run kStages - 1 steps ahead of the compute
// Stage slots per wave: the loads of step it + 1 run during step it. More
// slots keep more bytes in flight, but then the L2 evicts 128-byte lines
// before the wave of the neighbouring kv head (which reads the other half of
// the line) gets to them; two slots measured best.
template <int HS>
constexpr int stages_for() { return 2; }

template <int HS>
struct MfmaSmem {
  static constexpr int STAGE = StageGeo<HS>::BYTES;
  static constexpr int BUFB = 16 * HS * 4;                 // q' staging / epilogue (fp32 rows)
  static constexpr int NST = stages_for<HS>();
  static constexpr int MAINB = NST * STAGE > BUFB ? NST * STAGE : BUFB;
  alignas(16) unsigned char main[MAINB];                   // stages overlay the q / epilogue buffer
  float qsum[16];
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma(const void* g, void* l, int size) {
  switch (size) {
    case 1: __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 1, 0, 0); break;
    case 2: __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 2, 0, 0); break;
    case 4: __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 4, 0, 0); break;
    case 12: __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 12, 0, 0); break;
    default: __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 16, 0, 0); break;
  }
}

// Buffer-resource variant: uniform base in SGPRs, 32-bit per-lane offset;
// reads past num_records return 0 (never fault).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
template <int SIZE>
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* l) {
  if constexpr (SIZE == 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)l, 1, voff, 0, 0, 0);
  else if constexpr (SIZE == 2) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)l, 2, voff, 0, 0, 0);
  else if constexpr (SIZE == 4) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)l, 4, voff, 0, 0, 0);
  else if constexpr (SIZE == 12) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)l, 12, voff, 0, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)l, 16, voff, 0, 0, 0);
}

// s_waitcnt with only the vector-memory counter (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int HS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void attn_mfma_kernel(AttnArgs a, const int32_t* prefix) {
  using GG = Geo<HS>;
  using SG = StageGeo<HS>;
  constexpr int NK = GG::NK, NS = GG::NS, NVR = GG::NVR;
  constexpr int LP = (HS / 8) <= 8 ? 8 : ((HS / 8) <= 16 ? 16 : 32);   // lanes per row, chunk mapping
  constexpr int RPP = kWave / LP;                                       // rows per pass
  constexpr int HALF = HS / 2;
  constexpr int kStages = stages_for<HS>();
  __shared__ MfmaSmem<HS> smem_all[4];

  const int lane = threadIdx.x & 63;
  const int wv = uniform(threadIdx.x >> 6);           // wave index (uniform: LDS bases in SGPRs)
  MfmaSmem<HS>& sm = smem_all[wv];
  float* buf = reinterpret_cast<float*>(sm.main);
  const int n = lane & 15;          // MFMA column: query row of this lane
  const int q4 = lane >> 4;         // 0..3
  const int nkv = a.nkv;
  const int G = a.nq / nkv;
  const int gh = a.plan.gh;
  const int split = a.plan.split_tokens;
  const int total = uniform(prefix[a.num_seqs]);
  const int bsz = a.bs;
  const int bs_log2 = __builtin_ctz((unsigned)bsz);      // the planner sends only power-of-two pages here
  const int bs_mask = bsz - 1;
  const float inv_b = 1.0f / (float)a.b;
  // With num_kv_heads % 4 == 0 the 4 units of a workgroup are 4 kv heads of
  // one (sequence, query tile, head tile, split): the waves take the same
  // branches and run the same number of steps. A workgroup barrier per step
  // then keeps the waves of neighbouring kv heads (two per 128-byte line)
  // together, so each line comes from HBM once.
  const bool wg_sync = (nkv & 3) == 0;

  // lane constants of the chunk mapping (q setup and epilogue)
  const int cj = lane & (LP - 1);
  const bool c_on = cj < HS / 8;
  const uint32_t sbits = c_on ? sign_bits8(a.seed, cj) : 0u;
  uint32_t sx[4];
  sign_xor_bf16x8(sbits, sx);

  // lane byte offsets inside one half tile (relative to its first token row)
  const uint32_t tok_stride = (uint32_t)nkv * HALF;         // bytes between token rows of a page
  const uint32_t half_bytes = 16u * tok_stride;             // one half tile of a page
  const int64_t page_bytes = (int64_t)bsz * tok_stride;     // one page of one cache
  const int64_t page_rows = (int64_t)bsz * nkv;             // scale entries per page
  const uint32_t koff = (uint32_t)n * tok_stride + (uint32_t)q4 * (HS / 8);
  uint32_t vo[4];                                           // token 4*q4 + i, 32-bit column chunk n
#pragma unroll
  for (int i = 0; i < 4; ++i) vo[i] = (uint32_t)(4 * q4 + i) * tok_stride + 4u * (uint32_t)n;
  const uint32_t soff = (uint32_t)(lane & 15) * (uint32_t)nkv;   // scale elements
  const float* sc_base = lane < 32 ? a.k_scale : a.v_scale;
  const bool sc_half_b = (lane & 16) != 0;

  // Workgroups are dealt to the 8 XCDs round-robin (block b on XCD b % 8).
  // Unit quads 2k and 2k + 1 (kv heads 0-3 and 4-7 of one sequence split,
  // whose scale rows share 128-byte lines) go to blocks b and b + 8, which
  // share an XCD and its L2.
  const int nbk = gridDim.x, bk = blockIdx.x;
  const int pbk = bk < (nbk & ~15) ? ((bk & ~15) | ((bk & 7) << 1) | ((bk >> 3) & 1)) : bk;
  for (int u0 = pbk * 4; u0 < total; u0 += gridDim.x * 4) {
    const int u = u0 + wv;
    if (u >= total) continue;
    Unit un;
    if (!decode_unit(a, prefix, u, un)) continue;
    // the unit is the same for every lane of the wave
    const int us = uniform(un.s), ui0 = uniform(un.i0), uqbeg = uniform(un.qbeg);
    const int uqlen = uniform(un.qlen), uL = uniform(un.L), ug = uniform(un.g);
    const int uht = uniform(un.ht), usp = uniform(un.sp);
    const int h0 = ug * G + uht * gh;
    const int nh = min(gh, G - uht * gh);
    const int ntok = min(a.plan.tq, uqlen - ui0);
    const int pos0 = uL - uqlen + ui0;
    const int kend = pos0 + ntok;
    const int k0 = usp * split;
    const int k1 = min(k0 + split, kend);
    if (k0 >= k1 && usp > 0) continue;   // no keys for this tile in this split (the merge skips it)

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
        p = (p >= 0 && p < a.num_blocks) ? p : -1;
      }
      pg_lane = p;
    };
    const int nsteps = k1 > k0 ? (k1 - k0 + 31) / 32 : 0;
    if (nsteps > 0) load_pages(pg0);

    // ---- q' rows -> LDS (bf16 hi / lo, k-permuted) and their sums
#pragma unroll
    for (int ps = 0; ps < 16 / RPP; ++ps) {
      const int r = ps * RPP + lane / LP;
      const int ti = r / gh, hi = r - (r / gh) * gh;
      const bool rv = ti < ntok && hi < nh;
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (rv && c_on)
        w = *reinterpret_cast<const uint4*>(a.query + (int64_t)(uqbeg + ui0 + ti) * a.q_stride +
                                           (int64_t)(h0 + hi) * HS + 8 * cj);
      const uint32_t wd[4] = {w.x ^ sx[0], w.y ^ sx[1], w.z ^ sx[2], w.w ^ sx[3]};
      float v[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = bf16_lo(wd[k]);
        v[2 * k + 1] = bf16_hi(wd[k]);
      }
      fwht_b_ct<LP>(v, a.b, cj);
      float sum = 0.0f;
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // k-order of element offsets [0, 4, 1, 5, 2, 6, 3, 7]
        split_bf16x2(v[k] * a.scale_log2, v[k + 4] * a.scale_log2, hw[k], lw[k]);
        sum += (__uint_as_float(hw[k] << 16) + __uint_as_float(lw[k] << 16)) +
               (__uint_as_float(hw[k] & 0xFFFF0000u) + __uint_as_float(lw[k] & 0xFFFF0000u));
      }
      sum = group_sum_ct<LP>(c_on ? sum : 0.0f);
      if (c_on) {
        reinterpret_cast<uint4*>(buf)[(r * HS + 8 * cj) / 8] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        reinterpret_cast<uint4*>(buf)[(16 * HS + r * HS + 8 * cj) / 8] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
      if (cj == 0) sm.qsum[r] = sum;
    }
    __builtin_amdgcn_wave_barrier();
    uint4 qh[NK], ql[NK];
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      qh[s] = reinterpret_cast<const uint4*>(buf)[(n * HS + q4 * (HS / 4) + 8 * s) / 8];
      ql[s] = reinterpret_cast<const uint4*>(buf)[(16 * HS + n * HS + q4 * (HS / 4) + 8 * s) / 8];
    }
    const float qbias = 136.0f * sm.qsum[n];
    const int ti_n = n / gh, hi_n = n - (n / gh) * gh;
    const bool row_ok = ti_n < ntok && hi_n < nh;
    const int rpos = row_ok ? pos0 + ti_n : -1;
    const float row_add = row_ok ? 0.0f : -INFINITY;    // invalid rows never get weight
    // the staged q' has been read into registers before the stages overwrite it
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();

    f32x4_t acc[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t pacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    int okmask = 0;   // bit 2*slot: half A page valid, bit 2*slot+1: half B (wave-uniform)

    // issue the loads of step `it` into stage slot `it % kStages`; steps past
    // the end issue loads with an empty buffer range (they fetch nothing and
    // fill the slot with zeros, which is never read)
    auto issue = [&](unsigned char* __restrict__ st, int it) {
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
      // and the scale index of that row (kv head ug)
      const int64_t bya = (int64_t)pa * page_bytes + (int64_t)(offa * nkv + ug) * HALF;
      const int64_t byb = (int64_t)pb * page_bytes + (int64_t)(offb * nkv + ug) * HALF;
      int64_t rowa = (int64_t)pa * page_rows + offa * nkv + ug;
      int64_t rowb = (int64_t)pb * page_rows + offb * nkv + ug;
      const uint32_t nrec = dummy ? 0u : half_bytes;
      if (dummy) { rowa = 0; rowb = 0; }   // scale rows 0..15 of page 0: lines every wave keeps hot
      const __amdgpu_buffer_rsrc_t rk[2] = {rsrc(a.key_cache + bya, nrec),
                                            rsrc(a.key_cache + byb, nrec)};
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < SG::NKL; ++j) {
          unsigned char* dst = st + SG::K_OFF + h * SG::KHALF + j * SG::KREG;
          if constexpr (SG::KSZ == 16) dma_buf<16>(rk[h], koff + j * SG::KSZ, dst);
          else if constexpr (SG::KSZ == 12) dma_buf<12>(rk[h], koff + j * SG::KSZ, dst);
          else dma_buf<4>(rk[h], koff + j * SG::KSZ, dst);
        }
      const __amdgpu_buffer_rsrc_t rv[2] = {rsrc(a.value_cache + bya, nrec),
                                            rsrc(a.value_cache + byb, nrec)};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        unsigned char* dst = st + SG::V_OFF + i * SG::VBYTES_TOK;
        const uint32_t o = vo[i & 3];
#pragma unroll
        for (int r = 0; r < GG::RDW; ++r) dma_buf<4>(rv[i >> 2], o + 64 * r, dst + r * 256);
        if constexpr (GG::RUS) dma_buf<2>(rv[i >> 2], o - 2u * n + 64 * GG::RDW, dst + GG::RDW * 256);
        if constexpr (GG::RBY)
          dma_buf<1>(rv[i >> 2], o - 3u * n + 64 * GG::RDW + 32 * GG::RUS, dst + (GG::RDW + GG::RUS) * 256);
      }
      dma(sc_base + (sc_half_b ? rowb : rowa) + soff, st + SG::S_OFF, 4);
    };

    if (wg_sync) __builtin_amdgcn_s_barrier();
    if (nsteps > 0) {
#pragma unroll
      for (int i = 0; i < kStages - 1; ++i) issue(sm.main + i * SG::BYTES, i);
    }
    // `st` (read) and `wr` (filled for step it + kStages - 1) are distinct slots;
    // the restrict qualifiers let the compiler keep the lookahead loads in
    // flight across the reads of the current step.
    auto step = [&](const unsigned char* __restrict__ st, unsigned char* __restrict__ wr, int it) {
      const int slot = it % kStages;
      const int base = k0 + 32 * it;
      wait_vm<(kStages - 2) * SG::LOADS>();   // step `it` landed; later steps may be in flight
      if (wg_sync) __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue(wr, it + kStages - 1);            // into the slot step it - 1 used
      const bool oka = (okmask >> (2 * slot)) & 1, okb = (okmask >> (2 * slot + 1)) & 1;

      // K code words of this lane: token n, chunk q4, both half tiles
      uint32_t kw[2][NK];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned char* kr = st + SG::K_OFF + h * SG::KHALF;
        if constexpr (NK == 4) {
          const uint4 x = *reinterpret_cast<const uint4*>(kr + 16 * lane);
          kw[h][0] = x.x; kw[h][1] = x.y; kw[h][2] = x.z; kw[h][3] = x.w;
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
      // S^T for both half tiles (q' as hi + lo)
      f32x4_t sa = f32x4_t{0.f, 0.f, 0.f, 0.f}, sb = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        const uint4 ka = k_operand(kw[0][s]), kb = k_operand(kw[1][s]);
        sa = mfma_bf16(ka, qh[s], sa);
        sb = mfma_bf16(kb, qh[s], sb);
        sa = mfma_bf16(ka, ql[s], sa);
        sb = mfma_bf16(kb, ql[s], sb);
        __builtin_amdgcn_sched_barrier(0);   // keep one k-step's operands live at a time
      }
      const float* scl = reinterpret_cast<const float*>(st + SG::S_OFF);
      const float4 ksa = *reinterpret_cast<const float4*>(&scl[4 * q4]);
      const float4 ksb = *reinterpret_cast<const float4*>(&scl[16 + 4 * q4]);
      const float4 vsa = *reinterpret_cast<const float4*>(&scl[32 + 4 * q4]);
      const float4 vsb = *reinterpret_cast<const float4*>(&scl[48 + 4 * q4]);
      const float ks8[8] = {ksa.x, ksa.y, ksa.z, ksa.w, ksb.x, ksb.y, ksb.z, ksb.w};
      const float vs8[8] = {vsa.x, vsa.y, vsa.z, vsa.w, vsb.x, vsb.y, vsb.z, vsb.w};
      const float s8[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
      float lg[8];
      const bool full = base + 32 <= k1 && base + 31 <= pos0 && oka && okb;   // wave-uniform
      if (full) {
#pragma unroll
        for (int i = 0; i < 8; ++i) lg[i] = fmaf(s8[i] - qbias, ks8[i], row_add);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tok = base + (i < 4 ? 4 * q4 + i : 16 + 4 * q4 + (i - 4));
          const bool ok = tok < k1 && tok <= rpos && (i < 4 ? oka : okb);
          lg[i] = ok ? (s8[i] - qbias) * ks8[i] : -INFINITY;
        }
      }
      float mx = fmaxf(fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])),
                       fmaxf(fmaxf(lg[4], lg[5]), fmaxf(lg[6], lg[7])));
      mx = max_x16_x32(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      // a row that has seen no key yet has nothing to rescale
      const float alpha = m_run == -INFINITY ? 1.0f : fast_exp2(m_run - m_use);
      float psum_l = 0.0f;
      uint32_t pw[4], pl[4];
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float p0 = fast_exp2(lg[i] - m_use), p1 = fast_exp2(lg[i + 1] - m_use);
        psum_l += p0 + p1;
        split_bf16x2(p0 * vs8[i], p1 * vs8[i + 1], pw[i / 2], pl[i / 2]);
      }
      const uint4 ph4 = make_uint4(pw[0], pw[1], pw[2], pw[3]);
      const uint4 pl4 = make_uint4(pl[0], pl[1], pl[2], pl[3]);
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int i = 0; i < NS; ++i) acc[i] *= alpha;
        pacc *= alpha;
      }
      l_run = l_run * alpha + psum_l;
      m_run = m_new;

      // O'^T += V^T P^T, one n-step per V column of this lane's chunks
      int ns = 0;
#pragma unroll
      for (int r = 0; r < NVR; ++r) {
        int w, cb;
        v_region<HS>(r, w, cb);
        uint32_t x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const unsigned char* src = st + SG::V_OFF + i * SG::VBYTES_TOK;
          // sub-dword regions hold zero-extended words; their unused
          // nibbles are never selected below
          x[i] = reinterpret_cast<const uint32_t*>(src + r * 256)[lane];
        }
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          if (2 * jb >= w) break;
          const uint32_t t01 = pair_byte(x[0], x[1], jb);
          const uint32_t t23 = pair_byte(x[2], x[3], jb);
          const uint32_t t45 = pair_byte(x[4], x[5], jb);
          const uint32_t t67 = pair_byte(x[6], x[7], jb);
          const uint4 lo = make_uint4(nib2bf(t01), nib2bf(t23), nib2bf(t45), nib2bf(t67));
          const uint4 hi = make_uint4(nib2bf(t01 >> 4), nib2bf(t23 >> 4), nib2bf(t45 >> 4), nib2bf(t67 >> 4));
          acc[ns] = mfma_bf16(lo, ph4, acc[ns]);
          acc[ns + 1] = mfma_bf16(hi, ph4, acc[ns + 1]);
          acc[ns] = mfma_bf16(lo, pl4, acc[ns]);
          acc[ns + 1] = mfma_bf16(hi, pl4, acc[ns + 1]);
          ns += 2;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
      pacc = mfma_bf16(ones, ph4, pacc);
      pacc = mfma_bf16(ones, pl4, pacc);
    };
    for (int it = 0; it < nsteps; ++it)
      step(sm.main + (it % kStages) * SG::BYTES, sm.main + ((it + kStages - 1) % kStages) * SG::BYTES, it);
    wait_vm<0>();                             // no load may land in LDS after this point
    __builtin_amdgcn_wave_barrier();

    // ---- finish: l over the four lane quarters, remove the +136 offset
    l_run = sum_x16_x32(l_run);
    const float pbias = 136.0f * pacc[0];
    const int qrow = uqbeg + ui0 + ti_n;
    const int h = h0 + hi_n;
    if (a.plan.num_splits > 1) {
      if (row_ok) {
        const int64_t prow = ((int64_t)usp * a.num_q_tokens + qrow) * a.nq + h;
        float* dst = a.ws_o + prow * HS;
        int ns = 0;
#pragma unroll
        for (int r = 0; r < NVR; ++r) {
          int w, cb;
          v_region<HS>(r, w, cb);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            float* d = dst + cb + w * (4 * q4 + rr);
            if (w == 8) {
              reinterpret_cast<float4*>(d)[0] = make_float4(acc[ns][rr] - pbias, acc[ns + 1][rr] - pbias,
                                                            acc[ns + 2][rr] - pbias, acc[ns + 3][rr] - pbias);
              reinterpret_cast<float4*>(d)[1] = make_float4(acc[ns + 4][rr] - pbias, acc[ns + 5][rr] - pbias,
                                                            acc[ns + 6][rr] - pbias, acc[ns + 7][rr] - pbias);
            } else if (w == 4) {
              reinterpret_cast<float4*>(d)[0] = make_float4(acc[ns][rr] - pbias, acc[ns + 1][rr] - pbias,
                                                            acc[ns + 2][rr] - pbias, acc[ns + 3][rr] - pbias);
            } else {
              reinterpret_cast<float2*>(d)[0] = make_float2(acc[ns][rr] - pbias, acc[ns + 1][rr] - pbias);
            }
          }
          ns += w;
        }
        if (q4 == 0) {
          a.ws_ml[2 * prow] = m_run;
          a.ws_ml[2 * prow + 1] = l_run;
        }
      }
      continue;
    }
    // single split: normalize, stage the row in LDS, inverse rotation, store
    const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    __builtin_amdgcn_wave_barrier();
    {
      int ns = 0;
#pragma unroll
      for (int r = 0; r < NVR; ++r) {
        int w, cb;
        v_region<HS>(r, w, cb);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int c0 = cb + w * (4 * q4 + rr);
#pragma unroll
          for (int t = 0; t < 8; ++t)
            if (t < w) buf[n * HS + c0 + t] = (acc[ns + t][rr] - pbias) * inv_l;
        }
        ns += w;
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ps = 0; ps < 16 / RPP; ++ps) {
      const int r = ps * RPP + lane / LP;
      const int ti = r / gh, hi = r - (r / gh) * gh;
      const bool rv = ti < ntok && hi < nh;
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
      fwht_b_ct<LP>(o, a.b, cj);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = apply_sign(o[e] * inv_b, sbits, e);
      if (rv && c_on) {
        uint4 wo;
        wo.x = pack_bf16x2(o[0], o[1]);
        wo.y = pack_bf16x2(o[2], o[3]);
        wo.z = pack_bf16x2(o[4], o[5]);
        wo.w = pack_bf16x2(o[6], o[7]);
        *reinterpret_cast<uint4*>(a.out + ((int64_t)(uqbeg + ui0 + ti) * a.nq + h0 + hi) * HS + 8 * cj) = wo;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

static int g_num_cus = 0;

hipError_t launch_attn_mfma(const AttnArgs& a, int32_t* prefix, int64_t max_units, hipStream_t stream) {
  hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(1024), 0, stream, a, prefix);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g_num_cus == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      g_num_cus = cus;
    else
      g_num_cus = 256;
  }
  int64_t wgs = (max_units + 3) / 4;
  const int64_t cap = (int64_t)g_num_cus * 8;
  if (wgs > cap) wgs = cap;
  if (wgs < 1) wgs = 1;
  dim3 grid((unsigned)wgs), block(256);
  switch (a.hs) {
    case 64: hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, block, 0, stream, a, prefix); break;
    case 96: hipLaunchKernelGGL(attn_mfma_kernel<96>, grid, block, 0, stream, a, prefix); break;
    case 128: hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, block, 0, stream, a, prefix); break;
    case 192: hipLaunchKernelGGL(attn_mfma_kernel<192>, grid, block, 0, stream, a, prefix); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kv4
