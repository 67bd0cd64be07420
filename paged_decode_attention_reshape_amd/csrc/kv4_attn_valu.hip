// Read path (unified_attention_int4), vector-ALU split-KV kernel of libkv4,
// plus the cross-split log-sum-exp merge and output epilogue.
//
// Computes, per query row (query token, query head) and its kv head g:
//   q' = H.D.q (float32, never rounded), logit_j = k_scale_j (q' . code_j) *
//   softmax_scale / b, online softmax over the row's causal window, o' =
//   sum_j p_j v_scale_j code_V_j, out = D.H.o' / b rounded once to bf16 --
//   vLLM PR #62881 "[Bugfix][Test] Rotate KV into RHT domain in the INT4
//   unified attn test", Details / Root cause; divisor b per runguoli.com
//   "vLLM -- Attention Kernels & KV Cache Quantization", section "PR #56198";
//   metadata (block table, seq_lens, query_start_loc) per vLLM PR #40835
//   "[Feature] Triton INT4 per-token-head KV cache quantization", review
//   thread; the 2D / 3D (split along KV) launch choice mirrors the
//   seq_threshold_3D cases named in PR #62881, Validation.
//
// Mapping: one wave per (query tile, kv head, KV split). A KV token is handled
// by LPT = next_pow2(hs/8) lanes, each owning 8 elements (one 4-byte load of
// packed codes); a wave covers 64/LPT tokens per step. q' lives in registers
// in the same chunk layout, so dot products need only an LPT-lane reduction.
// Codes enter the arithmetic as u = code + 8 (an exact small integer taken
// from the nibble by masking and a byte-to-float conversion); the constant
// offset is removed once per dot product with the sum of q', and once per
// output element with the running sum of p * v_scale. Softmax runs in base 2
// with softmax_scale / b * log2(e) folded into q'.
#include <type_traits>

#include "kv4_device.hpp"
#include "kv4_launch.hpp"

namespace kv4 {

struct Tile {
  int s;        // sequence
  int i0;       // first query index of the tile inside the sequence
  int qbeg;     // first query row of the sequence
  int qlen;     // query_len of the sequence
  int L;        // seq_len, clamped to the page-table capacity
};

// Maps a query-tile index to (sequence, first query). With packed tiles,
// sequence s owns tiles qsl[s]/tq + s .. qsl[s+1]/tq + s (some may be empty).
__device__ __forceinline__ bool locate_tile(const AttnArgs& a, int64_t qt, Tile& t) {
  const int tq = a.plan.tq;
  int s;
  int64_t lt;
  if (a.plan.packed_tiles) {
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      const int64_t v = (int64_t)a.qsl[mid] / tq + mid;
      if (v <= qt) lo = mid; else hi = mid - 1;
    }
    s = lo;
    lt = qt - ((int64_t)a.qsl[s] / tq + s);
    if (lt < 0) return false;
  } else {
    s = (int)(qt / a.plan.tiles_per_seq);
    lt = qt - (int64_t)s * a.plan.tiles_per_seq;
  }
  if (s < 0 || s >= a.num_seqs) return false;
  int64_t qb, qe, L;
  seq_extent(a, s, qb, qe, L);
  const int qlen = (int)(qe - qb);
  if (lt * tq >= qlen) return false;
  t.s = s;
  t.i0 = (int)(lt * tq);
  t.qbeg = (int)qb;
  t.qlen = qlen;
  t.L = (int)L;
  return true;
}

// 8 packed int4 codes -> u = code + 8 as floats (exact).
__device__ __forceinline__ void codes_to_u(uint32_t w, float (&u)[8]) {
  const uint32_t x = w ^ 0x88888888u;
  const uint32_t lo = x & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6
  const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
  // (float)(byte k) lowers to v_cvt_f32_ubyte{k}
  u[0] = (float)(lo & 0xFFu);
  u[1] = (float)(hi & 0xFFu);
  u[2] = (float)((lo >> 8) & 0xFFu);
  u[3] = (float)((hi >> 8) & 0xFFu);
  u[4] = (float)((lo >> 16) & 0xFFu);
  u[5] = (float)((hi >> 16) & 0xFFu);
  u[6] = (float)(lo >> 24);
  u[7] = (float)(hi >> 24);
}

// 8 code bytes of the per-token-head modes -> exact float values:
// QM 1 two's-complement int8, QM 2 OCP e4m3fn (v_cvt_pk_f32_fp8).
template <int QM>
__device__ __forceinline__ void bytes_to_f(uint2 w, float (&u)[8]) {
  if constexpr (QM == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u[e] = (float)(int)(int8_t)(w.x >> (8 * e));
      u[e + 4] = (float)(int)(int8_t)(w.y >> (8 * e));
    }
  } else {
    const f32x2_t p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
    const f32x2_t p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
    const f32x2_t p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
    const f32x2_t p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
    u[0] = p0.x; u[1] = p0.y; u[2] = p1.x; u[3] = p1.y;
    u[4] = p2.x; u[5] = p2.y; u[6] = p3.x; u[7] = p3.y;
  }
}

// Store of one output row chunk without a rotation (per-token-head modes), bf16.
__device__ __forceinline__ void store_out_plain(const float (&o)[8], uint16_t* dst, bool do_store) {
  if (do_store) {
    uint4 w;
    w.x = pack_bf16x2(o[0], o[1]);
    w.y = pack_bf16x2(o[2], o[3]);
    w.z = pack_bf16x2(o[4], o[5]);
    w.w = pack_bf16x2(o[6], o[7]);
    *reinterpret_cast<uint4*>(dst) = w;
  }
}

// Inverse rotation and store of one output row chunk: o = D.H.o'/b, bf16.
// LPMAX > 0: at most LPMAX lanes per vector, with the lane distances fixed at
// compile time (no dispatch on them); LPMAX = 0: any b.
template <int LPMAX = 0>
__device__ __forceinline__ void store_out_row(float (&o)[8], int b, int jj, uint32_t sbits,
                                              float inv_b, uint16_t* dst, bool do_store) {
  if constexpr (LPMAX > 0) fwht_b_ct<LPMAX>(o, b, jj);
  else fwht_b(o, b, jj);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = apply_sign(o[e] * inv_b, sbits, e);
  if (do_store) {
    uint4 w;
    w.x = pack_bf16x2(o[0], o[1]);
    w.y = pack_bf16x2(o[2], o[3]);
    w.z = pack_bf16x2(o[4], o[5]);
    w.w = pack_bf16x2(o[6], o[7]);
    *reinterpret_cast<uint4*>(dst) = w;
  }
}

// QM: 0 int4 RHT cache; 1 / 2 int8 / fp8 per-token-head cache (no rotation).
template <int R, int QM>
__global__ __launch_bounds__(64) void attn_valu_kernel(AttnArgs a) {
  const int lane = threadIdx.x;
  const int hs = a.hs;
  const int LPT = next_pow2(hs >> 3);
  const int TPI = kWave / LPT;
  const int jj = lane & (LPT - 1);
  const int tg = lane / LPT;
  const bool lane_on = jj < (hs >> 3);

  const int G = a.nq / a.nkv;
  const int64_t qt = blockIdx.x / a.plan.n_head_tiles;
  const int ht = blockIdx.x - (int)qt * a.plan.n_head_tiles;
  const int g = blockIdx.y;
  const int sp = blockIdx.z;

  Tile t;
  if (!locate_tile(a, qt, t)) return;
  const int gh = a.plan.gh;
  const int h0 = g * G + ht * gh;
  const int nh = min(gh, G - ht * gh);
  const int ntok = min(a.plan.tq, t.qlen - t.i0);
  const int pos0 = t.L - t.qlen + t.i0;               // position of the tile's first query
  const int kend = pos0 + ntok;                       // keys [0, kend) are visible to some row
  // keys below the first query's sliding window are visible to no row
  const int kwin = a.window > 0 ? max(0, pos0 - a.window + 1) : 0;
  const int k0 = max(sp * a.plan.split_tokens, kwin);
  const int k1 = min(sp * a.plan.split_tokens + a.plan.split_tokens, kend);
  if (k0 >= k1 && a.plan.num_splits > 1) return;      // nothing here; the merge skips this split

  const uint32_t sbits = (QM == 0 && lane_on) ? sign_bits8(a.seed, jj) : 0u;
  uint32_t sx[4];
  sign_xor_bf16x8(sbits, sx);

  // ---- q' = H.D.q * (softmax_scale / b * log2 e), rows r = ti * gh + hi
  // (per-token-head modes: q' = q * softmax_scale * log2 e)
  float qv[R][8];
  float qsum[R];
  int rpos[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int ti = r / gh, hi = r - (r / gh) * gh;
    const bool rv = ti < ntok && hi < nh;
    rpos[r] = rv ? pos0 + ti : -1;
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (rv && lane_on) {
      const uint16_t* src = a.query + (int64_t)(t.qbeg + t.i0 + ti) * a.q_stride +
                            (int64_t)(h0 + hi) * hs + 8 * jj;
      w = *reinterpret_cast<const uint4*>(src);
    }
    const uint32_t wd[4] = {w.x ^ sx[0], w.y ^ sx[1], w.z ^ sx[2], w.w ^ sx[3]};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      qv[r][2 * k] = bf16_lo(wd[k]);
      qv[r][2 * k + 1] = bf16_hi(wd[k]);
    }
    if constexpr (QM == 0) fwht_b(qv[r], a.b, jj);
    float sum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[r][e] *= a.scale_log2;
      sum += qv[r][e];
    }
    qsum[r] = sum;
  }

  float acc[R][8];
  float m[R], l[R], psum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0f;
    psum[r] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.0f;
  }

  const int32_t* bt = a.block_table + (int64_t)t.s * a.max_blocks;

  for (int base = k0; base < k1; base += TPI) {
    const int tok = base + tg;
    bool valid = tok < k1;
    int64_t coff = 0, soff = 0;
    if (valid) {
      const int page = bt[tok / a.bs];
      valid = page >= 0 && page < a.num_blocks;
      KV4_DBG(!valid, KV4_DEBUG_PAGE);
      coff = a.lay.code_off(page, tok % a.bs, g);
      soff = a.lay.scale_off(page, tok % a.bs, g);
    }
    uint32_t kw = 0u, vw = 0u;
    uint2 kb = make_uint2(0u, 0u), vb = make_uint2(0u, 0u);
    float ks = 0.0f, vs = 0.0f;
    if (valid) {
      ks = a.k_scale[soff];
      vs = a.v_scale[soff];
      if (lane_on) {
        if constexpr (QM == 0) {
          kw = *reinterpret_cast<const uint32_t*>(a.key_cache + coff + 4 * jj);
          vw = *reinterpret_cast<const uint32_t*>(a.value_cache + coff + 4 * jj);
        } else {
          kb = *reinterpret_cast<const uint2*>(a.key_cache + coff + 8 * jj);
          vb = *reinterpret_cast<const uint2*>(a.value_cache + coff + 8 * jj);
        }
      }
    }
    float u[8];
    if constexpr (QM == 0) codes_to_u(kw, u);
    else bytes_to_f<QM>(kb, u);
    float logit[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float d = QM == 0 ? -8.0f * qsum[r] : 0.0f;    // int4: u = code + 8
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qv[r][e], u[e], d);
      d = lane_on ? d : 0.0f;
      logit[r] = group_sum(d, LPT) * ks;
      if (!valid || tok > rpos[r] || (a.window > 0 && tok <= rpos[r] - a.window)) logit[r] = -INFINITY;
    }
    if constexpr (QM == 0) codes_to_u(vw, u);
    else bytes_to_f<QM>(vb, u);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float mx = logit[r];
      for (int dd = LPT; dd < kWave; dd <<= 1) mx = fmaxf(mx, xor_lane_rt(mx, dd));
      const float m_new = fmaxf(m[r], mx);
      if (m_new == -INFINITY) continue;                      // wave-uniform
      const float p = fast_exp2(logit[r] - m_new);
      const float pv = p * vs;
      if (m_new != m[r]) {                                    // wave-uniform
        const float alpha = fast_exp2(m[r] - m_new);
        l[r] *= alpha;
        psum[r] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
        m[r] = m_new;
      }
      l[r] += p;
      psum[r] += pv;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(pv, u[e], acc[r][e]);
    }
  }

  // ---- combine the token groups of the wave
#pragma unroll
  for (int r = 0; r < R; ++r) {
    for (int dd = LPT; dd < kWave; dd <<= 1) {
      l[r] += xor_lane_rt(l[r], dd);
      psum[r] += xor_lane_rt(psum[r], dd);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] += xor_lane_rt(acc[r][e], dd);
    }
    if constexpr (QM == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(-8.0f, psum[r], acc[r][e]);
    }
  }

  const float inv_b = 1.0f / (float)a.b;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int ti = r / gh, hi = r - (r / gh) * gh;
    const bool rv = ti < ntok && hi < nh;
    const int64_t qrow = (int64_t)(t.qbeg + t.i0 + ti);
    const int h = h0 + hi;
    if (a.plan.num_splits == 1) {
      const float inv_l = l[r] > 0.0f ? 1.0f / l[r] : 0.0f;
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = acc[r][e] * inv_l;
      if constexpr (QM == 0)
        store_out_row(o, a.b, jj, sbits, inv_b, a.out + (qrow * a.nq + h) * hs + 8 * jj,
                      rv && lane_on && tg == 0);
      else
        store_out_plain(o, a.out + (qrow * a.nq + h) * hs + 8 * jj, rv && lane_on && tg == 0);
    } else if (rv && tg == 0) {
      const int64_t prow = ((int64_t)sp * a.num_q_tokens + qrow) * a.nq + h;
      if (lane_on) {
        float4* dst = reinterpret_cast<float4*>(a.ws_o + prow * hs + 8 * jj);
        dst[0] = make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
        dst[1] = make_float4(acc[r][4], acc[r][5], acc[r][6], acc[r][7]);
      }
      if (jj == 0) {
        a.ws_ml[2 * prow] = m[r];
        a.ws_ml[2 * prow + 1] = l[r];
      }
    }
  }
}

// Sequence of query token qtok and its step prefix (wave-uniform qtok).
struct RowSeq {
  int s;
  int64_t qb, qe, L, pf0, pf1, pftot;
};

__device__ __forceinline__ RowSeq row_sequence(const AttnArgs& a, int64_t qtok) {
  RowSeq q;
  // In single-token decode token t is nearly always sequence t: its
  // metadata is loaded with the check (one round trip), and the search runs
  // only if the guess is wrong.
  q.s = (int)(qtok < a.num_seqs ? qtok : a.num_seqs - 1);
  q.qb = a.qsl[q.s];
  q.qe = a.qsl[q.s + 1];
  q.L = a.seq_lens[q.s];
  q.pf0 = q.pf1 = q.pftot = 0;
  if (a.plan.sk) {
    q.pf0 = a.prefix[q.s];
    q.pf1 = a.prefix[q.s + 1];
    q.pftot = a.prefix[a.num_seqs];
  }
  if (!(q.qb <= qtok && qtok < q.qe)) {
    q.s = wave_search_le(a.qsl, a.num_seqs, qtok);
    q.qb = a.qsl[q.s];
    q.qe = a.qsl[q.s + 1];
    q.L = a.seq_lens[q.s];
    if (a.plan.sk) {
      q.pf0 = a.prefix[q.s];
      q.pf1 = a.prefix[q.s + 1];
    }
  }
  const int64_t cap = (int64_t)a.max_blocks * a.bs;
  q.L = q.L < 0 ? 0 : (q.L > cap ? cap : q.L);
  return q;
}

// RowSeq of a known sequence s (the compact row order below).
__device__ __forceinline__ RowSeq row_sequence_at(const AttnArgs& a, int s) {
  RowSeq q;
  q.s = s;
  q.qb = a.qsl[s];
  q.qe = a.qsl[s + 1];
  q.L = a.seq_lens[s];
  q.pf0 = q.pf1 = q.pftot = 0;
  if (a.plan.sk) {
    q.pf0 = a.prefix[s];
    q.pf1 = a.prefix[s + 1];
    q.pftot = a.prefix[a.num_seqs];
  }
  const int64_t cap = (int64_t)a.max_blocks * a.bs;
  q.L = q.L < 0 ? 0 : (q.L > cap ? cap : q.L);
  return q;
}

// The merge's rows. With a prefill kernel alongside, only the sequences this
// launch serves (at most q_hi queries each) have partials here: with compact
// rows they are enumerated as (sequence, query of the sequence < q_hi,
// head), so no row has to search for its sequence and the prefill rows are
// never visited; otherwise rows are (query token, head), and those of other
// launches' sequences are skipped. vrow -> (RowSeq, query token, head);
// false where the row has nothing to merge here.
__host__ __device__ inline int64_t merge_rows(const AttnArgs& a) {
  return compact_rows(a.plan) ? (int64_t)a.num_seqs * a.plan.q_hi * a.nq : a.num_q_tokens * a.nq;
}
__device__ __forceinline__ bool served_row(const AttnArgs& a, const RowSeq& q);
__device__ __forceinline__ bool merge_row(const AttnArgs& a, int64_t vrow, RowSeq& q, int64_t& qtok, int& h) {
  if (compact_rows(a.plan)) {
    const int64_t sq = (uint32_t)vrow / (uint32_t)a.nq;   // rows number fewer than 2^31 (checked on the host)
    h = (int)(vrow - sq * a.nq);
    const int dq = a.plan.q_hi;
    const int s = (int)(sq / dq), i = (int)(sq - (int64_t)s * dq);
    q = row_sequence_at(a, s);
    qtok = q.qb + i;
    return q.qb >= 0 && qtok < q.qe && qtok < a.num_q_tokens && served_row(a, q);
  }
  qtok = (uint32_t)vrow / (uint32_t)a.nq;
  h = (int)(vrow - qtok * a.nq);
  q = row_sequence(a, qtok);
  return served_row(a, q);
}

// Whether this launch serves the row's sequence (the same clamped test the
// planner kernels apply); every sequence without a prefill kernel.
__device__ __forceinline__ bool served_row(const AttnArgs& a, const RowSeq& q) {
  if (a.plan.pf_qlen <= 0) return true;
  int64_t qb = q.qb, qe = q.qe;
  qb = qb < 0 ? 0 : (qb > a.num_q_tokens ? a.num_q_tokens : qb);
  qe = qe < qb ? qb : (qe > a.num_q_tokens ? a.num_q_tokens : qe);
  return served_seq(a, qb, qe);
}

// The partials of output row `row` (query token qtok, query head h): nsp of
// them, partial k at workspace row k * pstride + pbase.
__device__ __forceinline__ void row_pieces(const AttnArgs& a, const RowSeq& q, int64_t qtok, int h, int64_t row,
                                           int& nsp, int64_t& pbase, int64_t& pstride) {
  nsp = 0;
  pbase = row;
  pstride = a.num_q_tokens * a.nq;
  if (compact_rows(a.plan) && !a.plan.sk) {
    // compact split rows (split, sequence, query of the sequence) of the
    // sequences left to the matrix-core kernel beside the prefill kernel
    pstride = (int64_t)a.num_seqs * a.plan.q_hi * a.nq;
    pbase = ((int64_t)q.s * a.plan.q_hi + (qtok - q.qb)) * a.nq + h;
  }
  if (a.plan.sk) {
    // stream-K: the workgroups whose step ranges cover this row's
    // (quad, sequence) steps [xs, xe) each left one piece, numbered
    // w + quad * num_seqs + s; workgroup w covers [w W / P, (w+1) W / P)
    const int quad = h / (a.nq / a.nkv) / a.plan.hpw / a.plan.wpb;
    const int64_t S = q.pftot;
    const int64_t W = (int64_t)a.plan.sk_quads * S;
    const int64_t P = (int64_t)a.plan.sk_grid < W ? (int64_t)a.plan.sk_grid : W;   // ranges, none empty
    const int64_t xs = (int64_t)quad * S + q.pf0, xe = (int64_t)quad * S + q.pf1;
    if (qtok >= q.qb && qtok < q.qe && xe > xs && W > 0) {
      // the range holding step x: the largest w with floor(w W / P) <= x
      const int64_t w0 = floor_div_small((xs + 1) * P - 1, W);
      const int64_t w1 = floor_div_small(xe * P - 1, W);
      nsp = (int)(w1 - w0 + 1);
      pbase = ((w0 + (int64_t)quad * a.num_seqs + q.s) * a.plan.tq + (qtok - q.qb)) * a.nq + h;
      pstride = (int64_t)a.plan.tq * a.nq;
    }
  } else if (qtok >= q.qb && qtok < q.qe) {
    const int64_t pos = q.L - (q.qe - q.qb) + (qtok - q.qb);
    if (pos >= 0) {
      const int64_t n = (pos + a.plan.split_tokens) / a.plan.split_tokens;   // ceil((pos+1)/split)
      nsp = (int)(n < a.plan.num_splits ? n : a.plan.num_splits);
      // sliding window: the splits before the one holding the row's first
      // visible key hold nothing for it (and may not have been written)
      if (a.window > 0 && pos - a.window + 1 > 0) {
        const int first = (int)((pos - a.window + 1) / a.plan.split_tokens);
        nsp -= first;
        pbase += (int64_t)first * pstride;
      }
    }
  }
}

// fold one partial (m2, l2, y) into the running (M, Ls, o)
__device__ __forceinline__ void lse_fold(float& M, float& Ls, float (&o)[8], float m2, float l2,
                                         const float (&y)[8]) {
  const float Mn = fmaxf(M, m2);
  if (Mn == -INFINITY) return;                   // both empty
  const float so = fast_exp2(M - Mn);            // 0 while M is -inf
  const float sn = fast_exp2(m2 - Mn);
  Ls = Ls * so + l2 * sn;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = o[e] * so + y[e] * sn;
  M = Mn;
}

// Merge of the split partials (log-sum-exp in base 2) and the output
// epilogue D.H(.)/b. One wave per output row (query token, query head): the
// wave holds NG = 64 / LP copies of the row (LP = next_pow2(hs/8) lanes of 8
// elements each); copy g folds splits g, g + NG, ... with four loads in flight,
// then a butterfly over the copies combines them. For calls with few rows
// (more waves share the latency-bound work).
template <int LP>
__global__ __launch_bounds__(256) void attn_reduce_kernel(AttnArgs a) {
  constexpr int NG = kWave / LP;
  const int hs = a.hs;
  const int lane = threadIdx.x & (kWave - 1);
  const int jj = lane & (LP - 1);
  const int grp = lane / LP;
  const bool lane_on = jj < (hs >> 3);
  // beside the prefill kernel, a launch that found no unit left no partial
  if (tile_class(a.plan) && a.prefix[a.num_seqs] == 0) return;
  const int64_t n_rows = merge_rows(a);
  const uint32_t sbits = (a.qm == 0 && lane_on) ? sign_bits8(a.seed, jj) : 0u;
  const float inv_b = 1.0f / (float)a.b;
  const int64_t wave0 = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t n_waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t vrow = wave0; vrow < n_rows; vrow += n_waves) {
    RowSeq q;
    int64_t qtok;
    int h;
    if (!merge_row(a, vrow, q, qtok, h)) continue;   // the prefill kernel's row, or none
    const int64_t row = qtok * a.nq + h;
    int nsp;
    int64_t pbase, pstride;
    row_pieces(a, q, qtok, h, row, nsp, pbase, pstride);
    float M = -INFINITY, Ls = 0.0f;
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int sp0 = grp; sp0 < nsp; sp0 += 4 * NG) {
      float mm[4], ll[4], y[4][8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int sp = sp0 + k * NG;
        mm[k] = -INFINITY;
        ll[k] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[k][e] = 0.0f;
        if (sp < nsp) {
          const int64_t prow = (int64_t)sp * pstride + pbase;
          mm[k] = a.ws_ml[2 * prow];
          ll[k] = a.ws_ml[2 * prow + 1];
          if (lane_on) {
            const float4* src = reinterpret_cast<const float4*>(a.ws_o + prow * hs + 8 * jj);
            const float4 x0 = src[0], x1 = src[1];
            y[k][0] = x0.x; y[k][1] = x0.y; y[k][2] = x0.z; y[k][3] = x0.w;
            y[k][4] = x1.x; y[k][5] = x1.y; y[k][6] = x1.z; y[k][7] = x1.w;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) lse_fold(M, Ls, o, mm[k], ll[k], y[k]);
    }
    // combine the NG copies (every lane of the wave takes part)
#pragma unroll
    for (int d = LP; d < kWave; d <<= 1) {
      const float m2 = xor_lane_rt(M, d), l2 = xor_lane_rt(Ls, d);
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = xor_lane_rt(o[e], d);
      lse_fold(M, Ls, o, m2, l2, y);
    }
    const float inv_l = Ls > 0.0f ? 1.0f / Ls : 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= inv_l;
    if (a.qm == 0) store_out_row<LP>(o, a.b, jj, sbits, inv_b, a.out + row * hs + 8 * jj, lane_on && grp == 0);
    else store_out_plain(o, a.out + row * hs + 8 * jj, lane_on && grp == 0);
  }
}

// The same merge for calls with many rows: each LP-lane group of a wave
// takes its own row, NG consecutive rows (one query token: num_q_heads is a
// multiple of NG) per wave, and folds the row's partials four loads at a
// time; no cross-group butterfly. A quarter of the waves (head size 128) of
// the one-row-per-wave form for the same rows.
template <int LP>
__global__ __launch_bounds__(256) void attn_reduce_rows_kernel(AttnArgs a) {
  constexpr int NG = kWave / LP;
  const int hs = a.hs;
  const int lane = threadIdx.x & (kWave - 1);
  const int jj = lane & (LP - 1);
  const int grp = lane / LP;
  const bool lane_on = jj < (hs >> 3);
  // beside the prefill kernel, a launch that found no unit left no partial
  if (tile_class(a.plan) && a.prefix[a.num_seqs] == 0) return;
  const int64_t n_units = merge_rows(a) / NG;
  const uint32_t sbits = (a.qm == 0 && lane_on) ? sign_bits8(a.seed, jj) : 0u;
  const float inv_b = 1.0f / (float)a.b;
  const int64_t wave0 = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t n_waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t u = wave0; u < n_units; u += n_waves) {
    // the wave's NG rows: consecutive heads of one query token
    RowSeq q;
    int64_t qtok;
    int h0;
    if (!merge_row(a, u * NG, q, qtok, h0)) continue;   // the prefill kernel's rows, or none
    const int h = h0 + grp;
    const int64_t row = qtok * a.nq + h;
    int nsp;
    int64_t pbase, pstride;
    row_pieces(a, q, qtok, h, row, nsp, pbase, pstride);
    float M = -INFINITY, Ls = 0.0f;
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int sp0 = 0; sp0 < nsp; sp0 += 4) {
      float mm[4], ll[4], y[4][8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int sp = sp0 + k;
        mm[k] = -INFINITY;
        ll[k] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[k][e] = 0.0f;
        if (sp < nsp) {
          const int64_t prow = (int64_t)sp * pstride + pbase;
          mm[k] = a.ws_ml[2 * prow];
          ll[k] = a.ws_ml[2 * prow + 1];
          if (lane_on) {
            const float4* src = reinterpret_cast<const float4*>(a.ws_o + prow * hs + 8 * jj);
            const float4 x0 = src[0], x1 = src[1];
            y[k][0] = x0.x; y[k][1] = x0.y; y[k][2] = x0.z; y[k][3] = x0.w;
            y[k][4] = x1.x; y[k][5] = x1.y; y[k][6] = x1.z; y[k][7] = x1.w;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) lse_fold(M, Ls, o, mm[k], ll[k], y[k]);
    }
    const float inv_l = Ls > 0.0f ? 1.0f / Ls : 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= inv_l;
    // the epilogue's lane exchanges stay inside each LP-lane group
    if (a.qm == 0) store_out_row<LP>(o, a.b, jj, sbits, inv_b, a.out + row * hs + 8 * jj, lane_on);
    else store_out_plain(o, a.out + row * hs + 8 * jj, lane_on);
  }
}

hipError_t launch_attn_valu(const AttnArgs& a, hipStream_t stream) {
  const int64_t gx = a.plan.n_qtiles * a.plan.n_head_tiles;
  dim3 grid((unsigned)gx, (unsigned)a.nkv, (unsigned)a.plan.num_splits), block(64);
  auto go = [&](auto qm) {
    constexpr int QM = decltype(qm)::value;
    switch (a.plan.rows) {
      case 1: hipLaunchKernelGGL((attn_valu_kernel<1, QM>), grid, block, 0, stream, a); break;
      case 2: hipLaunchKernelGGL((attn_valu_kernel<2, QM>), grid, block, 0, stream, a); break;
      case 4: hipLaunchKernelGGL((attn_valu_kernel<4, QM>), grid, block, 0, stream, a); break;
      default: hipLaunchKernelGGL((attn_valu_kernel<8, QM>), grid, block, 0, stream, a); break;
    }
  };
  switch (a.qm) {
    case 0: go(std::integral_constant<int, 0>()); break;
    case 1: go(std::integral_constant<int, 1>()); break;
    case 2: go(std::integral_constant<int, 2>()); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_reduce(const AttnArgs& a, hipStream_t stream) {
  const int LP = host_next_pow2(a.hs / 8);
  const int NG = kWave / LP;
  const int64_t rows = merge_rows(a);
  // one row per lane group where the caller asks for it and a wave's NG rows
  // share one query token
  if (a.reduce_rows && a.nq % NG == 0) {
    const int64_t units = rows / NG;                 // waves (grid-stride beyond 2^22)
    const int64_t blocks = std::min<int64_t>((units + 3) / 4, a.plan.wg_cap > 0 ? a.plan.wg_cap : (int64_t)1 << 20);
    dim3 grid((unsigned)std::max<int64_t>(blocks, 1)), block(256);
    switch (LP) {
      case 1: hipLaunchKernelGGL(attn_reduce_rows_kernel<1>, grid, block, 0, stream, a); break;
      case 2: hipLaunchKernelGGL(attn_reduce_rows_kernel<2>, grid, block, 0, stream, a); break;
      case 4: hipLaunchKernelGGL(attn_reduce_rows_kernel<4>, grid, block, 0, stream, a); break;
      case 8: hipLaunchKernelGGL(attn_reduce_rows_kernel<8>, grid, block, 0, stream, a); break;
      case 16: hipLaunchKernelGGL(attn_reduce_rows_kernel<16>, grid, block, 0, stream, a); break;
      case 32: hipLaunchKernelGGL(attn_reduce_rows_kernel<32>, grid, block, 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int64_t blocks =
      std::min<int64_t>((rows + 3) / 4, a.plan.wg_cap > 0 ? a.plan.wg_cap : (int64_t)1 << 20);   // one wave per row
  dim3 grid((unsigned)std::max<int64_t>(blocks, 1)), block(256);
  switch (LP) {
    case 1: hipLaunchKernelGGL(attn_reduce_kernel<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(attn_reduce_kernel<2>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(attn_reduce_kernel<4>, grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(attn_reduce_kernel<8>, grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL(attn_reduce_kernel<16>, grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL(attn_reduce_kernel<32>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

KV4_DEBUG_ACCESSOR(debug_flags_valu)

}  // namespace kv4
