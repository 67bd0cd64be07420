// Host-side launch interface between the C ABI (kv4_api.cpp) and the HIP
// kernel translation units of libkv4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kv4_device.hpp"

namespace kv4 {

inline int host_next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Addressing of a paged cache: the code bytes of (page p, token slot t of
// the page, kv head h) start p * blk + t * tok + h * head bytes after the
// cache base, and its scale sits p * sblk + t * stok + h * shead floats after
// the scale base. The packed layout (C code bytes per row): blk = bs * nkv *
// C, tok = nkv * C, head = C, sblk = bs * nkv, stok = nkv, shead = 1.
struct CacheLayout {
  int64_t blk, tok, head;
  int64_t sblk, stok, shead;
  __host__ __device__ int64_t code_off(int64_t page, int64_t t, int64_t h) const {
    return page * blk + t * tok + h * head;
  }
  __host__ __device__ int64_t scale_off(int64_t page, int64_t t, int64_t h) const {
    return page * sblk + t * stok + h * shead;
  }
};

inline CacheLayout packed_layout(int nkv, int code_bytes, int bs) {
  CacheLayout l;
  l.head = code_bytes;
  l.tok = (int64_t)nkv * code_bytes;
  l.blk = (int64_t)bs * l.tok;
  l.shead = 1;
  l.stok = nkv;
  l.sblk = (int64_t)bs * nkv;
  return l;
}

struct WriteArgs {
  const uint16_t* key;
  const uint16_t* value;
  int64_t key_stride;    // elements between token rows
  int64_t value_stride;
  uint8_t* key_cache;
  uint8_t* value_cache;
  float* k_scale;
  float* v_scale;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int64_t num_slots;     // num_blocks * block_size
  int nkv;
  int hs;
  int b;
  uint64_t seed;
  int qm;                // 0: int4 RHT; 1: int8 per-token-head; 2: fp8 (e4m3fn) per-token-head
  int bs;                // block size
  int bs_shift;          // log2(bs) if bs is a power of two, else -1
  CacheLayout lay;
  int slices;            // head-vector slices a wave loads before computing any (2 or 4; set by launch_write)
};

struct DequantArgs {
  const uint8_t* cache;
  const float* scale;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int64_t num_slots;
  int nkv;
  int hs;
  int b;
  uint64_t seed;
  int inverse_rotate;
  float* out;
  int qm;                // as WriteArgs
  int bs;
  int bs_shift;
  CacheLayout lay;
};

// Waves per workgroup of the matrix-core kernel at (kv heads per wave, cache
// mode, head size), as the kernels are built; the planner's stream-K cut
// uses the same value. Four heads per wave, and int8 / fp8 at head size 192
// (12 KB stages), take two waves so that more workgroups fit a CU's LDS.
constexpr int mfma_waves_per_block(int hpw, int qm, int hs) {
  return (hpw == 4 || (qm != 0 && hs >= 192)) ? 2 : 4;
}

// Sequences the prefill kernel's in-kernel unit prefix covers (four per
// thread of its 256); calls with more run without the prefill kernel.
constexpr int kPfMaxSeqs = 1024;
// Query tiles per prefill workgroup: sequences with more than this many tiles
// of queries go to the prefill kernel.
constexpr int kPfUnitTiles = 4;

// Work decomposition of one attention call (chosen on the host from host-known
// sizes only; no device data is read).
struct AttnPlan {
  int path;            // 0 = VALU split-KV kernel, 1 = MFMA kernel
  int tq;              // query tokens per tile
  int gh;              // query heads (of one kv head's group) per tile
  int rows;            // tq * gh rounded up to the kernel's row count
  int n_head_tiles;    // ceil(group / gh)
  int packed_tiles;    // 1: tiles found by search over query_start_loc
  int64_t n_qtiles;    // tiles of query tokens (grid, before head tiles)
  int tiles_per_seq;   // uniform mode: tiles per sequence
  int split_tokens;    // KV tokens per split
  int num_splits;      // splits in the grid (1 = no partials)
  int hpw;             // MFMA path: kv heads per wave (1, 2 or 4; > 1 only for single-token decode)
  int wpb;             // MFMA path: waves per workgroup
  int sk;              // MFMA single-token decode: stream-K partition instead of splits
  int sk_quads;        // stream-K: kv head groups / waves per workgroup
  int sk_pcap;         // stream-K: most workgroups (sizes the workspace)
  int sk_grid;         // stream-K: workgroups launched (set at launch)
  int sk_per_cu;       // stream-K: at most this many workgroups per CU (0: as many as fit)
  int vjh;             // MFMA, head size 128, hpw > 1: V staged per head (heads not adjacent)
  int rb;              // MFMA, int4, hpw 1: 16-row MFMA blocks per wave (1 or 2)
  int fused_plan;      // MFMA: the kernel computes the sequences' prefix itself (set at launch)
  // Chunked-prefill sequences (int4, query length >= pf_qlen) run on the
  // prefill kernel. 0 = none. Beside it the other sequences are split by
  // query length into launches of the kernels above (and the merge), each
  // serving q_lo <= query_len <= q_hi (< pf_qlen) and skipping the rest.
  int pf_qlen;
  int pf_tq;           // prefill: query tokens per wave tile (32 rows / group)
  int pf_grid;         // prefill: workgroups launched (a multiple of 8, >= its units)
  int q_lo, q_hi;      // beside the prefill kernel: the query lengths this launch serves
  // beside the prefill kernel: split partial and merge rows are (query token,
  // head) as without it, where the batch has fewer query tokens than
  // sequences x q_hi; otherwise (sequence, query of the sequence < q_hi, head)
  int tok_rows;
  // most workgroups of this launch and of its merge (0: as many as the work
  // asks); both loop over their units grid-stride
  int wg_cap;
};

// Whether a plan's split partial and merge rows are the compact (sequence,
// query of the sequence, head) rows of a launch beside the prefill kernel.
__host__ __device__ inline bool compact_rows(const AttnPlan& p) { return p.pf_qlen > 0 && !p.tok_rows; }

struct AttnArgs {
  const uint16_t* query;
  int64_t q_stride;
  const uint8_t* key_cache;
  const uint8_t* value_cache;
  const float* k_scale;
  const float* v_scale;
  int64_t num_blocks;
  const int32_t* block_table;
  int max_blocks;
  const int32_t* seq_lens;
  const int32_t* qsl;
  int num_seqs;
  int64_t num_q_tokens;
  int max_query_len;
  int max_seq_len;
  int nq;
  int nkv;
  int hs;
  int b;
  int bs;
  uint64_t seed;
  float scale_log2;    // softmax_scale / b * log2(e)
  uint16_t* out;
  float* ws_o;         // [num_splits][num_q_tokens][nq][hs]   (split only)
  float* ws_ml;        // [num_splits][num_q_tokens][nq][2]    (split only)
                       // stream-K: [sk_pcap + quads * num_seqs][nq][hs] and [..][nq][2]
  const int32_t* prefix;   // MFMA path: device plan output (stream-K: first KV step per sequence)
  int qm;                  // 0: int4 RHT cache; 1 / 2: int8 / fp8 per-token-head cache (no rotation)
  CacheLayout lay;         // shared by the K and V caches and their scales
  int window;              // sliding window: the query at position p sees keys (p - window, p]; 0 = none
  int reduce_rows;         // merge: one row per lane group (few partials per row) instead of per wave
  int code_nt;             // MFMA path: K/V code loads carry the non-temporal hint (head size 128 kernels)
  AttnPlan plan;
};

// Query range [qb, qe) and cached length L of sequence s, clamped to what the
// call's buffers hold (the kernels read nothing outside them whatever the
// metadata says).
__device__ __forceinline__ void seq_extent(const AttnArgs& a, int s, int64_t& qb, int64_t& qe, int64_t& L) {
  qb = a.qsl[s];
  qe = a.qsl[s + 1];
  KV4_DBG(qb < 0 || qe < qb || qe > a.num_q_tokens, KV4_DEBUG_QSL);
  KV4_DBG(a.seq_lens[s] < 0 || (int64_t)a.seq_lens[s] > (int64_t)a.max_blocks * a.bs, KV4_DEBUG_SEQLEN);
  qb = qb < 0 ? 0 : (qb > a.num_q_tokens ? a.num_q_tokens : qb);
  qe = qe < qb ? qb : (qe > a.num_q_tokens ? a.num_q_tokens : qe);
  L = a.seq_lens[s];
  const int64_t cap = (int64_t)a.max_blocks * a.bs;
  L = L < 0 ? 0 : (L > cap ? cap : L);
}

// Whether a sequence with the (clamped) query range [qb, qe) belongs to the
// prefill kernel.
__device__ __forceinline__ bool prefill_seq(const AttnArgs& a, int64_t qb, int64_t qe) {
  return a.plan.pf_qlen > 0 && qe - qb >= a.plan.pf_qlen;
}

// Whether a launch of the kernels beside the prefill kernel serves the
// sequence with the (clamped) query range [qb, qe): every sequence without
// a prefill kernel, else those with q_lo <= query_len <= q_hi.
__device__ __forceinline__ bool served_seq(const AttnArgs& a, int64_t qb, int64_t qe) {
  return a.plan.pf_qlen <= 0 || (qe - qb >= a.plan.q_lo && qe - qb <= a.plan.q_hi);
}

// Whether a plan is the launch of the 2 .. Q-query sequences beside the
// prefill kernel.
__host__ __device__ inline bool tile_class(const AttnPlan& p) { return p.pf_qlen > 0 && p.q_lo > 1; }

// Debug builds: the KV4_DEBUG_* words of the kernel files (0 in release).
uint32_t debug_flags_write(bool clear);
uint32_t debug_flags_mfma(bool clear);
uint32_t debug_flags_prefill(bool clear);
uint32_t debug_flags_valu(bool clear);

hipError_t launch_write(const WriteArgs& a, hipStream_t stream);
hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream);
hipError_t launch_attn_valu(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_reduce(const AttnArgs& a, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, int64_t bytes, unsigned int* sink, int grid, hipStream_t stream);
// Device plan (work units per sequence, exclusive prefix into `prefix`,
// num_seqs + 1 ints) followed by the matrix-core attention kernel.
// In stream-K mode it sets a.plan.sk_grid, which the merge needs.
hipError_t launch_attn_mfma(AttnArgs& a, int32_t* prefix, int64_t max_units, hipStream_t stream);
// The chunked-prefill kernel (a.plan.pf_qlen > 0): every query row of the
// prefill sequences, written to the output directly.
hipError_t launch_attn_prefill(AttnArgs& a, hipStream_t stream);

}  // namespace kv4
