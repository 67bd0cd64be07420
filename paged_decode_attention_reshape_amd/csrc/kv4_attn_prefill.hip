// Read path, chunked-prefill sequences (int4 RHT cache, head size 128): the
// query rows of sequences with many new tokens, on the matrix cores with the
// K/V stream shared by a whole workgroup.
//
// Math per query row as in the other attention kernels (vLLM PR #62881
// "[Bugfix][Test] Rotate KV into RHT domain in the INT4 unified attn test",
// Details / Root cause; divisor b per runguoli.com "vLLM -- Attention Kernels
// & KV Cache Quantization", section "PR #56198"): q' = H.D.q, logit_j =
// k_scale_j (q' . code_j) softmax_scale / b, causal (and sliding-window)
// online softmax, o' = sum p_j v_scale_j code_V_j, out = D.H.o'/b. Prefill
// and decode rows of one batch are served by one call (vLLM PR #40835 review:
// one unified attention entry point for both).
//
// Why a kernel of its own. A prefill chunk's rows all read the same keys, so
// the work is a dense contraction: 4 hs flops per (query head, visible key)
// against 136 bytes per (kv head, key). What bounds it is how much matrix
// and vector work each staged K/V byte feeds:
//   * A workgroup takes four consecutive query tiles of one (sequence, kv
//     head): 4 x 32 MFMA rows (query tokens x the GQA group). Its key range
//     is cut in two halves, and each (tile, half) is one of its eight waves
//     (two per SIMD, so one wave's vector work hides the other's matrix
//     work). Each 32-token K/V step of a half is loaded once into that
//     half's four-slot LDS ring (direct buffer -> LDS loads, spread over its
//     four waves, two steps ahead) and read by all four; one workgroup
//     barrier per two steps.
//   * The two halves of a tile are merged in LDS at the end (log-sum-exp),
//     so every row is finished on chip and written once as bf16: no fp32
//     partials in memory, no merge kernel.
//   * Units are numbered so that the workgroups of one (sequence, kv head)
//     run on one XCD (workgroup b runs on XCD b % 8) and share its L2, the
//     latest tiles (most keys) first.
// Per step and wave the arithmetic is that of the two-row-block form of the
// decode/multi-token kernel: S^T = K . Q'^T on v_mfma_f32_16x16x32_bf16 with
// q' as a bf16 hi + lo pair, exact nibble -> bf16 / fp16 operands, the K code
// offset 136 taken out through the accumulator's start value (-136 sum q'),
// O'^T = V^T P^T on v_mfma_f32_16x16x32_f16 with p * v_scale under a per-step
// power of two, and the V code offset 72 removed with a ones-MFMA.
#include <cstdio>
#include <cstdlib>

#include "kv4_device.hpp"
#include "kv4_launch.hpp"
#include "kv4_mfma_ops.hpp"

namespace kv4 {

namespace {

constexpr int kPfTiles = kPfUnitTiles;          // query tiles per workgroup
constexpr int kPfHalves = 2;                    // key-range halves per tile
constexpr int kPfWaves = kPfTiles * kPfHalves;  // waves per workgroup
constexpr int kPfSteps = 2;                     // key steps per workgroup barrier
constexpr int kPfSlots = 2 * kPfSteps;          // ring slots per half: kPfSteps being read, kPfSteps in flight
constexpr int kPfSeqsPerThread = (kPfMaxSeqs + 64 * kPfWaves - 1) / (64 * kPfWaves);

// One ring slot: one 32-token step of one kv head (head size 128).
//   K  half tile h (16 tokens): 1 KB at K_OFF + 1024 h; lane l's 16 bytes
//      are code bytes [16 (l >> 4), +16) of token l & 15
//   V  half tile h: 1 KB at V_OFF + 1024 h, the 16 token rows of 64 bytes
//   S  64 floats: k_scale of token l & 15 of half tile (l >> 4) & 1 for
//      l < 32, v_scale of the same tokens for l >= 32
struct PfSlot {
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 2048;
  static constexpr int S_OFF = 4096;
  static constexpr int BYTES = 4352;
};

// Workgroup units of a sequence with the (clamped) query range [qb, qe):
// ceil(tiles / kPfTiles) per kv head for the prefill kernel's sequences, 0
// for the others.
__device__ __forceinline__ int pf_units(const AttnArgs& a, int64_t qb, int64_t qe) {
  if (!prefill_seq(a, qb, qe)) return 0;
  const int64_t tiles = (qe - qb + a.plan.pf_tq - 1) / a.plan.pf_tq;
  return (int)((tiles + kPfTiles - 1) / kPfTiles) * a.nkv;
}

// Exclusive prefix of pf_units over the sequences into lds[0 .. num_seqs]
// (lds[num_seqs] = total), by the threads of the workgroup: thread t owns
// sequences [k t, k t + k), k = kPfSeqsPerThread, so the metadata comes in
// one round trip. lds needs num_seqs + 1 + kPfWaves ints.
__device__ int pf_prefix(const AttnArgs& a, int32_t* lds) {
  constexpr int K = kPfSeqsPerThread;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = a.num_seqs;
  int u[K];
  int own = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int s = K * tid + k;
    u[k] = 0;
    if (s < n) {
      int64_t qb, qe, L;
      seq_extent(a, s, qb, qe, L);
      u[k] = pf_units(a, qb, qe);
    }
    own += u[k];
  }
  int x = own;   // inclusive scan of the per-thread sums inside the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  int32_t* wave_tot = lds + n + 1;
  if (lane == 63) wave_tot[wv] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kPfWaves; ++i) {
    before += i < wv ? wave_tot[i] : 0;
    all += wave_tot[i];
  }
  int run = before + x - own;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int s = K * tid + k;
    if (s < n) lds[s] = run;
    run += u[k];
  }
  if (tid == 0) lds[n] = all;
  __syncthreads();
  return all;
}

}  // namespace

// WIN: built with the sliding-window terms.
template <bool WIN>
__global__ __launch_bounds__(64 * kPfWaves) __attribute__((amdgpu_waves_per_eu(2))) void attn_prefill_kernel(
    AttnArgs a) {
  constexpr int HS = 128;
  constexpr int NK = HS / 32;        // QK k-steps
  constexpr int NRB = 2;             // 16-row MFMA blocks per wave
  constexpr int ROWS = 16 * NRB;
  constexpr int LP = 16;             // lanes per row in the q' / output passes (8 elements each)
  constexpr int RPP = kWave / LP;    // rows per pass
  constexpr int HALF = HS / 2;       // code bytes per token row of one kv head
  constexpr int D = kPfSlots - kPfSteps;   // steps of lookahead
  using SL = PfSlot;
  // one K/V ring per key half; per wave one 8 KB buffer: the q' rows of one
  // row block (bf16 hi, then lo) at the start, the second half's partial
  // rows (fp32) for the merge, then the output rows (fp32); the unit prefix
  // overlays the buffers before any of that
  __shared__ __attribute__((aligned(16))) unsigned char ring[kPfHalves][kPfSlots * SL::BYTES];
  __shared__ __attribute__((aligned(16))) float wbuf[kPfWaves][16 * HS];
  __shared__ float qsum_s[kPfWaves][ROWS];
  __shared__ float mstat[kPfTiles][ROWS], lstat[kPfTiles][ROWS], pstat[kPfTiles][ROWS];
  static_assert(sizeof(wbuf) >= (kPfMaxSeqs + 1 + kPfWaves) * sizeof(int32_t), "prefix overlay");

  const int lane = threadIdx.x & 63;
  const int wv = uniform(threadIdx.x >> 6);
  const int tl = wv & (kPfTiles - 1);   // query tile of the workgroup
  const int kh = wv / kPfTiles;         // key half
  const int role = wv & 3;              // loads of its half: K half tile 0 (+ scales), K 1, V 0, V 1

  // ---- the unit of this workgroup
  int32_t* pfx = reinterpret_cast<int32_t*>(&wbuf[0][0]);
  const int total = pf_prefix(a, pfx);
  // workgroup b runs on XCD b % 8: units [x C, (x + 1) C) go to XCD x
  const int C = (total + 7) / 8;
  const int bk = blockIdx.x;
  const int u = (bk & 7) * C + (bk >> 3);
  if ((bk >> 3) >= C || u >= total) return;   // the whole workgroup leaves together
  const int s = wave_search_le(pfx, a.num_seqs, u);
  const int rem = u - pfx[s];
  __syncthreads();                            // the prefix is read; wbuf is free

  int64_t qb64, qe64, L64;
  seq_extent(a, s, qb64, qe64, L64);
  const int qb = uniform((int)qb64), qlen = uniform((int)(qe64 - qb64)), L = uniform((int)L64);
  const int G = a.nq / a.nkv;
  const int tq = a.plan.pf_tq;
  const int ntiles = (qlen + tq - 1) / tq;
  const int ntw = (ntiles + kPfTiles - 1) / kPfTiles;
  const int g = rem / ntw;                            // kv head
  const int jw = ntw - 1 - (rem - g * ntw);           // workgroup tile: latest first
  const int i0 = (jw * kPfTiles + tl) * tq;           // this wave's first query of the sequence
  const int ntok = max(0, min(tq, qlen - i0));
  const int pos0 = L - qlen + i0;                     // position of query i0
  // the workgroup's keys: up to its last query's position, from the 32-step
  // holding its first query's window start; steps [0, n0) are half 0's,
  // [n0, nsteps) half 1's
  const int wq0 = jw * kPfTiles * tq, wq1 = min(qlen, (jw + 1) * kPfTiles * tq);
  const int kw1 = max(0, min(L, L - qlen + wq1));
  const int kw0 = WIN ? (max(0, L - qlen + wq0 - a.window + 1) & ~31) : 0;
  const int nsteps = kw1 > kw0 ? (kw1 - kw0 + 31) / 32 : 0;
  const int n0 = (nsteps + 1) / 2;
  const int hs0 = kh * n0;                            // this half's first step
  const int hn = kh == 0 ? n0 : nsteps - n0;          // and its number of steps
  // this wave's keys
  const int k1w = ntok > 0 ? max(0, min(L, pos0 + ntok)) : 0;
  const int k0w = WIN ? max(0, pos0 - a.window + 1) : 0;
  const int win = WIN ? a.window : INT_MAX;
  const int wlo = WIN ? pos0 + ntok - a.window : INT_MIN;   // keys >= wlo are in every row's window

  const int n = lane & 15;          // MFMA column: query row of this lane
  const int q4 = lane >> 4;
  const int cj = lane & (LP - 1);
  const uint32_t sbits = sign_bits8(a.seed, cj);
  uint32_t sx[4];
  sign_xor_bf16x8(sbits, sx);
  const int bs_log2 = __builtin_ctz((unsigned)a.bs);
  const int bs_mask = a.bs - 1;
  const float inv_b = 1.0f / (float)a.b;

  // ---- K/V ring loads of this half's step `it` into slot it % kPfSlots of
  // its ring, one or two loads per wave (its role). Steps past the half's
  // end load with an empty buffer range (zeros, never read).
  const uint32_t tok_stride = (uint32_t)a.lay.tok;
  const uint32_t half_bytes = 16u * tok_stride;
  const int64_t head_off = (int64_t)g * a.lay.head;
  const uint32_t koff = (uint32_t)n * tok_stride + (uint32_t)q4 * 16u;
  const uint32_t vsrc = (uint32_t)(lane >> 2) * tok_stride + 16u * (uint32_t)(lane & 3);
  const int64_t soff = (int64_t)(lane & 15) * a.lay.stok + (int64_t)g * a.lay.shead;
  const float* sc_base = lane < 32 ? a.k_scale : a.v_scale;
  const bool sc_half_b = (lane & 16) != 0;
  const int32_t* bt = a.block_table + (int64_t)s * a.max_blocks;
  const int npages = kw1 > 0 ? ((kw1 - 1) >> bs_log2) + 1 : 0;
  int pg0 = 0, pg_lane = -1;
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
  if (hn > 0) load_pages((kw0 + 32 * hs0) >> bs_log2);
  unsigned char* const myring = ring[kh];
  int okmask = 0;   // bit 2 slot: half tile A page valid, bit 2 slot + 1: half tile B (wave-uniform)
  auto issue = [&](unsigned char* __restrict__ st, int it) {
    const int slot = it % kPfSlots;
    const bool dummy = it >= hn;
    const int base = kw0 + 32 * (hs0 + (dummy ? 0 : it));
    const bool b_in = base + 16 < kw1;
    const int pga = base >> bs_log2;
    const int pgb = b_in ? (base + 16) >> bs_log2 : pga;
    int ia = pga - pg0, ib = pgb - pg0;
    if (ia < 0 || ib >= 64) {             // the next 64 pages of the table
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
    const uint32_t nrec = dummy ? 0u : half_bytes;
    const int ht = role & 1;              // half tile of this wave's code load
    const int64_t by = (int64_t)(ht ? pb : pa) * a.lay.blk + (int64_t)(ht ? offb : offa) * tok_stride + head_off;
    if (role < 2) {
      dma_buf<16>(rsrc(a.key_cache + by, nrec), koff, st + SL::K_OFF + ht * 1024);
      if (role == 0) {
        int64_t row = sc_half_b ? (int64_t)pb * a.lay.sblk + (int64_t)offb * a.lay.stok
                                : (int64_t)pa * a.lay.sblk + (int64_t)offa * a.lay.stok;
        if (dummy) row = 0;               // rows of page 0: in bounds, never read
        dma(sc_base + row + soff, st + SL::S_OFF, 4);
      }
    } else {
      dma_buf<16>(rsrc(a.value_cache + by, nrec), vsrc, st + SL::V_OFF + ht * 1024);
    }
  };

  // ---- q' rows of the tile, computed by its first-half wave: bf16 hi / lo
  // pairs (k-permuted), kept in LDS for the whole key walk and read per
  // k-step by both waves of the tile: hi rows in wbuf[t], lo rows in
  // wbuf[t + 4]. 16-byte chunk c of row n sits at chunk c ^ n, so the 16
  // lanes of a read hit 16 different bank groups.
  float* buf = wbuf[wv];
  const unsigned char* qhi = reinterpret_cast<const unsigned char*>(wbuf[tl]);
  const unsigned char* qlo = reinterpret_cast<const unsigned char*>(wbuf[tl + kPfTiles]);
  float qbias[NRB], row_add[NRB];
  int rpos[NRB];
  uint4 qhr[NRB][NK];   // hi rows of this lane's two MFMA rows, per k-step (the lo rows stay in LDS)
  if (kh == 0) {
    uint4* hi_rows = reinterpret_cast<uint4*>(wbuf[tl]);
    uint4* lo_rows = reinterpret_cast<uint4*>(wbuf[tl + kPfTiles]);
#pragma unroll
    for (int ps = 0; ps < ROWS / RPP; ++ps) {
      const int r = ps * RPP + lane / LP;          // row of the tile
      const int ti = r / G, hi = r - (r / G) * G;
      const bool rv = ti < ntok;
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (rv)
        w = *reinterpret_cast<const uint4*>(a.query + (int64_t)(qb + i0 + ti) * a.q_stride +
                                           (int64_t)(g * G + hi) * HS + 8 * cj);
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
      sum = group_sum_ct<LP>(sum);
      hi_rows[r * (HS / 8) + (cj ^ (r & 15))] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      lo_rows[r * (HS / 8) + (cj ^ (r & 15))] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      if (cj == 0) qsum_s[tl][r] = sum;
    }
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int rn = 16 * rb + n;
#pragma unroll
    for (int k = 0; k < NK; ++k) qhr[rb][k] = *reinterpret_cast<const uint4*>(qhi + rb * (16 * HS * 2) + (((uint32_t)n * (HS * 2) + 16u * (uint32_t)((4 * q4) ^ n)) ^ (16u * k)));
    const int ti = rn / G;
    const bool ok = ti < ntok;
    // the K operands are 136 + code: the accumulator starts at -136 sum(q')
    qbias[rb] = -136.0f * qsum_s[tl][rn];
    rpos[rb] = ok ? pos0 + ti : -1;
    row_add[rb] = ok ? 0.0f : -INFINITY;   // rows past the tile never get weight
  }
  // this lane's q' chunk offsets: row 16 rb + n, chunk (4 q4 + k) ^ n
  const uint32_t qlo_off = (uint32_t)n * (HS * 2) + 16u * (uint32_t)((4 * q4) ^ n);

  f32x4_t acc[NRB][8];
  f32x4_t pacc[NRB];
  float m_run[NRB], l_run[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[rb][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    pacc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.0f;
  }
  float e_run = -100.0f;   // running v_scale exponent (see the softmax step)
  uint32_t vrd[4];         // LDS offset of token 4 q4 + i, code word n, in a V half tile
#pragma unroll
  for (int i = 0; i < 4; ++i) vrd[i] = (uint32_t)((4 * q4 + i) * HALF) + 4u * (uint32_t)n;
  // S^T = K . Q'^T of one step, both half tiles (q' as hi + lo); lane n
  // keeps the 8 logits of its row (in sa / sb until the softmax takes them)
  f32x4_t sa[NRB], sb[NRB];
  auto qk = [&](const unsigned char* __restrict__ st) {
    uint32_t kw[2][NK];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 x = *reinterpret_cast<const uint4*>(st + SL::K_OFF + h * 1024 + 16 * lane);
      kw[h][0] = x.x; kw[h][1] = x.y; kw[h][2] = x.z; kw[h][3] = x.w;
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      sa[rb] = f32x4_t{qbias[rb], qbias[rb], qbias[rb], qbias[rb]};
      sb[rb] = sa[rb];
    }
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const uint4 ka = k_operand(kw[0][k]), kb = k_operand(kw[1][k]);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        // chunk (4 q4 + k) ^ n = ((4 q4) ^ n) ^ k: k only flips the low two bits
        const uint32_t qo = rb * (16 * HS * 2) + (qlo_off ^ (16u * k));
        const uint4 qh = qhr[rb][k];
        const uint4 ql = *reinterpret_cast<const uint4*>(qlo + qo);
        sa[rb] = mfma_bf16(ka, qh, sa[rb]);
        sb[rb] = mfma_bf16(kb, qh, sb[rb]);
        sa[rb] = mfma_bf16(ka, ql, sa[rb]);
        sb[rb] = mfma_bf16(kb, ql, sb[rb]);
      }
      __builtin_amdgcn_sched_barrier(0);   // one k-step's operands live at a time
    }
  };
  // mask, online softmax and O'^T += V^T P^T of step `it` (its logits in sa / sb)
  auto smpv = [&](const unsigned char* __restrict__ st, int it) {
    const int slot = it % kPfSlots;
    const int base = kw0 + 32 * (hs0 + it);
    const bool oka = (okmask >> (2 * slot)) & 1, okb = (okmask >> (2 * slot + 1)) & 1;
    const float* scl = reinterpret_cast<const float*>(st + SL::S_OFF);
    const float4 ksa = *reinterpret_cast<const float4*>(&scl[4 * q4]);
    const float4 ksb = *reinterpret_cast<const float4*>(&scl[16 + 4 * q4]);
    const float4 vsa = *reinterpret_cast<const float4*>(&scl[32 + 4 * q4]);
    const float4 vsb = *reinterpret_cast<const float4*>(&scl[48 + 4 * q4]);
    const float ks8[8] = {ksa.x, ksa.y, ksa.z, ksa.w, ksb.x, ksb.y, ksb.z, ksb.w};
    const float vs8[8] = {vsa.x, vsa.y, vsa.z, vsa.w, vsb.x, vsb.y, vsb.z, vsb.w};
    // every row sees all 32 keys (wave-uniform)
    const bool full = base + 31 <= pos0 && (!WIN || base >= wlo) && oka && okb;
    float lg[NRB][8], mx[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float s8[8] = {sa[rb][0], sa[rb][1], sa[rb][2], sa[rb][3], sb[rb][0], sb[rb][1], sb[rb][2], sb[rb][3]};
      if (full) {
#pragma unroll
        for (int i = 0; i < 8; ++i) lg[rb][i] = fmaf(s8[i], ks8[i], row_add[rb]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tok = base + (i < 4 ? 4 * q4 + i : 16 + 4 * q4 + (i - 4));
          const bool ok = tok <= rpos[rb] && (!WIN || tok > rpos[rb] - win) && (i < 4 ? oka : okb);
          lg[rb][i] = ok ? s8[i] * ks8[i] : -INFINITY;
        }
      }
      mx[rb] = fmaxf(fmaxf(fmaxf(lg[rb][0], lg[rb][1]), fmaxf(lg[rb][2], lg[rb][3])),
                     fmaxf(fmaxf(lg[rb][4], lg[rb][5]), fmaxf(lg[rb][6], lg[rb][7])));
      mx[rb] = max_x16_x32(mx[rb]);
    }
    // p * v_scale enters the matrix cores as one fp16 under 2^-e, e = (the
    // exponent of the step's largest v_scale) - 11 kept as a running maximum:
    // below 2^12 and clear of fp16 subnormals; acc, pacc and l carry the
    // scale 2^-(m + e), m the running logit maximum.
    float vmx = fmaxf(fmaxf(fmaxf(vs8[0], vs8[1]), fmaxf(vs8[2], vs8[3])),
                      fmaxf(fmaxf(vs8[4], vs8[5]), fmaxf(vs8[6], vs8[7])));
    vmx = max_x16_x32(vmx);
    const float e_step = fmaxf((float)((int)((__float_as_uint(vmx) >> 23) & 0xFFu) - 138), -100.0f);
    const float e_new = fmaxf(e_run, e_step);
    uint4 ph4[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      // lazy maximum: a row keeps its running maximum until a step's logits
      // exceed it by more than 3 (p <= 8 then; p * v_scale * 2^-e < 2^15
      // still fits fp16), so most steps rescale nothing
      const float m_new = mx[rb] > m_run[rb] + 3.0f ? mx[rb] : m_run[rb];
      const float big_m = (m_new == -INFINITY ? 0.0f : m_new) + e_new;
      // a row that has seen no key yet has nothing to rescale
      const float alpha = m_run[rb] == -INFINITY ? 1.0f : fast_exp2(m_run[rb] + e_run - big_m);
      float psum = 0.0f;
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float p0 = fast_exp2(lg[rb][i] - big_m), p1 = fast_exp2(lg[rb][i + 1] - big_m);
        psum += p0 + p1;
        pw[i / 2] = pack_f16x2(p0 * vs8[i], p1 * vs8[i + 1]);
      }
      ph4[rb] = make_uint4(pw[0], pw[1], pw[2], pw[3]);
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[rb][i] *= alpha;
        pacc[rb] *= alpha;
      }
      l_run[rb] = l_run[rb] * alpha + psum;
      m_run[rb] = m_new;
    }
    e_run = e_new;
    // O'^T += V^T P^T: lane (n, q4) holds code word n (columns 8n .. 8n + 7)
    // of tokens 4 q4 + i of both halves
    uint32_t x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = *reinterpret_cast<const uint32_t*>(st + SL::V_OFF + (i >> 2) * 1024 + vrd[i & 3]);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const uint32_t t01 = pair_byte(x[0], x[1], jb);
      const uint32_t t23 = pair_byte(x[2], x[3], jb);
      const uint32_t t45 = pair_byte(x[4], x[5], jb);
      const uint32_t t67 = pair_byte(x[6], x[7], jb);
      // low nibbles (column 2 jb) moved up to bits 4-7; high nibbles in place
      const uint4 lo = make_uint4(nib2h(t01 << 4), nib2h(t23 << 4), nib2h(t45 << 4), nib2h(t67 << 4));
      const uint4 hi = make_uint4(nib2h(t01), nib2h(t23), nib2h(t45), nib2h(t67));
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        acc[rb][2 * jb] = mfma_f16(lo, ph4[rb], acc[rb][2 * jb]);
        acc[rb][2 * jb + 1] = mfma_f16(hi, ph4[rb], acc[rb][2 * jb + 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);   // fp16 1.0
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) pacc[rb] = mfma_f16(ones, ph4[rb], pacc[rb]);
  };

  // ---- the key walk: one workgroup barrier per pair of steps. At the
  // barrier before steps it and it + 1 every wave has finished steps it - 2
  // and it - 1, so their slots take steps it + D and it + D + 1. (One
  // barrier per step measured 4 % slower: at each barrier the waves that
  // finish first idle while their SIMD partner finishes alone; three or
  // four steps per barrier, with their larger rings, gained less than two.)
  // (Running the two waves of a SIMD out of phase, one on QK while the other
  // is on the softmax, measured slower: the two code paths cost more
  // register moves than the overlap won.)
  //
  // Every ring load and every ring read of the walk sits in `step`, whose
  // slot pointers are restrict parameters: the compiler then knows that the
  // loads in flight (into other slots) do not feed the reads, and keeps them
  // in flight instead of draining the load counter before each read; the
  // counts waited for below order them. The first calls only load (the
  // prologue), through the same instructions.
  static_assert(kPfSteps == 2 && D % kPfSteps == 0, "two steps per call");
  auto step = [&](unsigned char* __restrict__ w0, unsigned char* __restrict__ w1,
                  const unsigned char* __restrict__ r0, const unsigned char* __restrict__ r1, int it) {
    issue(w0, it + D);
    issue(w1, it + D + 1);
    if (it < 0) return;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = it + j;
      const int base = kw0 + 32 * (hs0 + i);
      if (i < hn && base < k1w && base + 32 > k0w) {   // wave-uniform
        qk(j ? r1 : r0);
        smpv(j ? r1 : r0, i);
      }
    }
  };
  // slot of step i; the empty asm keeps the offset an opaque scalar, so the
  // compiler adds it to the few per-lane offsets at each read instead of
  // carrying a per-lane address per slot and read kind in registers
  auto slot_at = [&](int i) {
    uint32_t off = (uint32_t)((i + 2 * kPfSlots) % kPfSlots) * SL::BYTES;
    asm volatile("" : "+s"(off));
    return myring + off;
  };
  for (int it = -D; it < n0; it += kPfSteps) {
    if (it >= 0) {
      // this wave's loads of steps it and it + 1 have landed (those of the
      // D - 2 later steps may still be in flight)
      if (role == 0) wait_vm<2 * (D - kPfSteps)>();
      else wait_vm<D - kPfSteps>();
      __builtin_amdgcn_s_waitcnt(0xC07F);   // and this wave's LDS reads of steps it - 2, it - 1 have returned
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    step(slot_at(it + D), slot_at(it + D + 1), slot_at(it), slot_at(it + 1), it);
  }
  wait_vm<0>();   // no load may land in LDS after this point
  __syncthreads();   // every wave is done with the q' lo rows (wbuf[t + 4] takes the merge partials)

  // ---- merge the key halves of each tile (log-sum-exp: acc, pacc and l of
  // a half carry the scale 2^-(m + e) of its own running maximum m and v_scale
  // exponent e), then the finish: the V offset (64 + u = 72 + code) out
  // through the sum of the rounded P, normalize, inverse rotation D.H(.)/b,
  // bf16 rows out
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    float l = sum_x16_x32(l_run[rb]);
    float me = m_run[rb] == -INFINITY ? -INFINITY : m_run[rb] + e_run;
    float pa0 = pacc[rb][0];
    if (kh == 1) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int c0 = 8 * (4 * q4 + rr);
#pragma unroll
        for (int t = 0; t < 8; ++t) buf[n * HS + c0 + t] = acc[rb][t][rr];
      }
      if (q4 == 0) {
        mstat[tl][16 * rb + n] = me;
        lstat[tl][16 * rb + n] = l;
        pstat[tl][16 * rb + n] = pa0;
      }
    }
    __syncthreads();
    if (kh == 0) {
      const float* pb = wbuf[wv + kPfTiles];
      const float me1 = mstat[tl][16 * rb + n];
      const float mt = fmaxf(me, me1);
      const float f0 = mt == -INFINITY ? 0.0f : fast_exp2(me - mt);
      const float f1 = mt == -INFINITY ? 0.0f : fast_exp2(me1 - mt);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int c0 = 8 * (4 * q4 + rr);
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[rb][t][rr] = acc[rb][t][rr] * f0 + pb[n * HS + c0 + t] * f1;
      }
      l = l * f0 + lstat[tl][16 * rb + n] * f1;
      pa0 = pa0 * f0 + pstat[tl][16 * rb + n] * f1;
      const float pbias = 72.0f * pa0;
      const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int c0 = 8 * (4 * q4 + rr);
#pragma unroll
        for (int t = 0; t < 8; ++t) buf[n * HS + c0 + t] = (acc[rb][t][rr] - pbias) * inv_l;
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int ps = 0; ps < 16 / RPP; ++ps) {
        const int rl = ps * RPP + lane / LP;
        const int r = 16 * rb + rl;
        const int ti = r / G, hi = r - (r / G) * G;
        float o[8];
        const float4 x0 = reinterpret_cast<const float4*>(buf)[(rl * HS + 8 * cj) / 4];
        const float4 x1 = reinterpret_cast<const float4*>(buf)[(rl * HS + 8 * cj) / 4 + 1];
        o[0] = x0.x; o[1] = x0.y; o[2] = x0.z; o[3] = x0.w;
        o[4] = x1.x; o[5] = x1.y; o[6] = x1.z; o[7] = x1.w;
        fwht_b_ct<LP>(o, a.b, cj);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = apply_sign(o[e] * inv_b, sbits, e);
        if (ti < ntok) {
          uint4 wo;
          wo.x = pack_bf16x2(o[0], o[1]);
          wo.y = pack_bf16x2(o[2], o[3]);
          wo.z = pack_bf16x2(o[4], o[5]);
          wo.w = pack_bf16x2(o[6], o[7]);
          *reinterpret_cast<uint4*>(a.out + ((int64_t)(qb + i0 + ti) * a.nq + g * G + hi) * HS + 8 * cj) = wo;
        }
      }
    }
    __syncthreads();   // the partner buffers and stats are rewritten for the next row block
  }
}

// Workgroups for the prefill kernel's units, a multiple of 8 at least their
// number: each prefill sequence (>= pf_qlen queries) has ceil(q / (4 tq))
// <= q / (4 tq) + 1 units per kv head, and there are at most
// min(num_seqs, num_q_tokens / pf_qlen) of them.
int64_t prefill_grid(const AttnArgs& a) {
  const int64_t npf = std::min<int64_t>(a.num_seqs, a.num_q_tokens / a.plan.pf_qlen);
  const int64_t units = (a.num_q_tokens / ((int64_t)kPfTiles * a.plan.pf_tq) + 1 + npf) * a.nkv;
  return (units + 7) / 8 * 8;
}

hipError_t launch_attn_prefill(AttnArgs& a, hipStream_t stream) {
  if (a.plan.pf_qlen <= 0) return hipSuccess;
  if (a.hs != 128 || a.qm != 0 || a.num_seqs > kPfMaxSeqs || a.plan.pf_tq < 1 ||
      a.plan.pf_tq * (a.nq / a.nkv) > 32)
    return hipErrorInvalidValue;   // the planner sends only these shapes
  const int64_t grid = prefill_grid(a);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  a.plan.pf_grid = (int)grid;
  const dim3 blk(64 * kPfWaves);
  if (a.window > 0) hipLaunchKernelGGL(attn_prefill_kernel<true>, dim3((unsigned)grid), blk, 0, stream, a);
  else hipLaunchKernelGGL(attn_prefill_kernel<false>, dim3((unsigned)grid), blk, 0, stream, a);
  return hipGetLastError();
}

KV4_DEBUG_ACCESSOR(debug_flags_prefill)

}  // namespace kv4
