// libkv4 C ABI: argument validation, work planning and kernel launches.
// The declarations and their contracts are in include/kv4.h.
#include "kv4.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <vector>
#include <string>

#include "kv4_launch.hpp"

// Device memory of kv4_paged_attention_noalloc: its split partials and
// sequence prefix, in place of a caller workspace. Every GPU the library runs
// on holds its own copy from the library's first use there until the process
// ends. In host code `scratch` names a host-side stand-in: only the address
// hipGetSymbolAddress returns for the current device may reach a kernel.
static __device__ __align__(256) unsigned char scratch[KV4_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

kv4_status fail(kv4_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kv4_status fail(kv4_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

kv4_status ok() {
  g_last_error.clear();
  return KV4_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// b == 0 asks for the rule's value: the largest power of two dividing head_size.
kv4_status check_head(int32_t head_size, int32_t& b) {
  if (head_size < 8 || head_size > 256 || head_size % 8 != 0)
    return fail(KV4_EINVAL, "head_size must be a multiple of 8 in [8, 256], got %d", head_size);
  const int32_t want = head_size & -head_size;
  if (b == 0) b = want;
  if (b != want)
    return fail(KV4_EINVAL,
                "b must be the largest power of two dividing head_size (%d for head_size %d), got %d",
                want, head_size, b);
  return KV4_OK;
}

kv4_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KV4_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

long env_long(const char* name, long dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  char* end = nullptr;
  const long x = std::strtol(v, &end, 10);
  return (end && *end == 0) ? x : dflt;
}

constexpr int kRowsMax = 8;             // query rows per VALU wave
constexpr int kMfmaRows = 16;           // query rows per MFMA tile
constexpr int64_t kTargetUnitsValu = 2048;
constexpr int64_t kTargetUnitsMfma = 16384;
constexpr int kMinSplit = 256;
constexpr int kSkMaxGrid = 2048;        // stream-K workgroups at most (8 per CU of a 256-CU GPU)
constexpr int kSkMinSteps = 16;         // stream-K: KV steps per workgroup at least ...
constexpr int kSkMinGrid = 512;         // ... unless that leaves fewer than 2 workgroups per CU (256 CUs)
constexpr bool kPthMfma = true;        // matrix-core kernels for the int8 / fp8 caches
constexpr int64_t kReduceRowsMinWaves = 2048;   // merge: one row per lane group from this many waves
// Workgroups of the launch (and of the merge) of the 2 .. Q-query sequences
// beside the prefill kernel. It is sized for every query tile of the batch,
// yet often serves few sequences or none (a chunked-prefill batch of long
// chunks and decodes), and while the prefill kernel holds most CUs a full
// grid of workgroups that find no unit still queues for the few free CUs.
constexpr int kTileLaunchWgs = 512;

bool mfma_head_size(int hs) { return hs == 64 || hs == 96 || hs == 128 || hs == 192 || hs == 256; }
// int4 head sizes 80 and 112 (b = 16) run on the kernels of 96 and 128 with
// the 16 missing columns zero in q' (one kv head per wave)
bool mfma_padded_head_size(int hs) { return hs == 80 || hs == 112; }

// Kv heads one matrix-core wave serves by default at a head size: each head
// adds a 2-slot LDS stage (about 8.7 KB at head size 128), and larger stages
// cut the waves a CU holds below what hides the load latency (measured best:
// 2 at 64, 96 and 128; 1 at 192 and 256).
int mfma_hpw_max(int hs) { return (hs >= 192 || mfma_padded_head_size(hs)) ? 1 : 2; }

// Host planner: depends only on host-known sizes (and the KV4_SPLIT_TOKENS /
// KV4_FORCE_PATH overrides used by tests), so the workspace size and the
// launch agree. Path 1 (matrix cores) is used where the query block is dense
// (GQA group > 1 or query_len > 1), the head size is a multiple of 32 the
// kernel is built for, and pages hold a power-of-two number (>= 16) of tokens.
// The query lengths one launch of the kernels beside the prefill kernel
// serves, and the prefill kernel's own threshold and tile.
struct PfClass {
  int pf_qlen, pf_tq, q_lo, q_hi;
};

// single: the plan without the prefill kernel. min_split: the launch of a
// class beside it splits no finer than this many tokens.
kv4_status make_plan_for(int qm, int64_t num_q_tokens, int32_t num_seqs, int32_t nq, int32_t nkv, int32_t hs,
              int32_t max_query_len, int32_t max_seq_len, int32_t block_size, const kv4::CacheLayout& lay,
              kv4::AttnPlan& p, const PfClass* cls, PfClass* pf_out, bool single = false, int min_split = 0) {
  std::memset(&p, 0, sizeof(p));
  if (pf_out) *pf_out = PfClass{0, 0, 0, 0};
  const int G = nq / nkv;
  const int64_t code_bytes = qm ? hs : hs / 2;
  // the matrix-core kernel moves 16-byte pieces with 32-bit offsets inside a
  // 16-token half tile (head sizes 80 / 112: 4- and 12-byte pieces, so
  // 4-byte strides); heads of one token row side by side (and their scales)
  // let one wave serve several kv heads
  const int dma_align = (qm == 0 && mfma_padded_head_size(hs)) ? 4 : 16;
  const bool lay_dma = lay.blk % dma_align == 0 && lay.tok % dma_align == 0 && lay.head % dma_align == 0 &&
                       lay.tok <= (INT32_MAX - 4096) / 16;
  const bool lay_contig = lay.head == code_bytes && lay.shead == 1;
  const bool hs_ok = (mfma_head_size(hs) && (qm == 0 || kPthMfma)) || (qm == 0 && mfma_padded_head_size(hs));
  const bool mfma_ok = hs_ok && lay_dma && block_size % 16 == 0 && (block_size & (block_size - 1)) == 0;
  // The matrix-core kernel wherever the shape allows it: even single-query
  // decode with one query head per kv head (one busy MFMA row of 16 unless a
  // wave serves several kv heads) streams the cache about 4x faster through
  // its LDS pipeline than the vector kernel.
  bool mfma = mfma_ok;
  if (const char* f = std::getenv("KV4_FORCE_PATH")) {
    if (!std::strcmp(f, "valu")) mfma = false;
    if (!std::strcmp(f, "mfma")) mfma = mfma_ok;
  }
  p.path = mfma ? 1 : 0;
  // Chunked prefill (int4, head size 128, GQA group <= 32): with the prefill
  // kernel on, the sequences with more than Q = 4 tiles of 32 / G queries (at
  // least one whole prefill workgroup) go to it, whose workgroups share each
  // staged K/V step among four tiles and walk every tile's whole key range.
  // The others run on the kernels above in two launches: the single-query
  // sequences as decode (two kv heads per wave, stream-K where the heads
  // allow), not as 32-row tiles with one query in them; those with 2 .. Q
  // queries as tiles (and key splits), where the prefill kernel would walk
  // their whole context in two halves with far fewer waves.
  //
  // KV4_PREFILL: 0 off, 1 on wherever the shape allows, otherwise (default)
  // on where a sequence may have more than Q queries and the tokens beyond
  // one per sequence could fill 128 prefill workgroups ((T - S) x kv heads >=
  // 128 Q). Measured (attention call, cache read from HBM; prefill path
  // against the single-kernel plan): Qwen2.5-1.5B shape (group 6) 4 chunks of
  // 512 + 60 decodes 121 against 159 us, 2 x 2048 + 30 decodes 267 / 332;
  // Llama-3-8B shape (group 4) 2 x 512 + 128 decodes over 4k-32k contexts
  // 529 / 816, 8 x 256 + 16 decodes 159 / 210, 1 x 512 + 64 four-query
  // sequences 505 / 522. Left on the single-kernel plan: Qwen shape 1 x 512 +
  // 60 decodes (106 / 98 with the prefill kernel: one chunk's workgroups take
  // a whole walk of its context however many CUs are free), 4 x 64 + 60
  // decodes (94 / 63), 1 x 512 + 64 four-query sequences (108 / 75).
  p.pf_qlen = 0;
  if (cls) {
    // a launch beside the prefill kernel: its class of query lengths
    p.pf_qlen = cls->pf_qlen;
    p.pf_tq = cls->pf_tq;
    p.q_lo = cls->q_lo;
    p.q_hi = cls->q_hi;
    // partial rows per split: the fewer of sequences x q_hi and query tokens
    p.tok_rows = num_q_tokens < (int64_t)num_seqs * cls->q_hi ? 1 : 0;
    max_query_len = cls->q_hi;
  } else if (!single) {
    const long pf_mode = env_long("KV4_PREFILL", 2);
    if (mfma && qm == 0 && hs == 128 && G <= 32 && num_seqs <= kv4::kPfMaxSeqs && pf_mode != 0) {
      const int pf_tq = 32 / G;
      const int Q = kv4::kPfUnitTiles * pf_tq;
      const bool chunky = (num_q_tokens - num_seqs) * nkv >= 128LL * Q;
      if (max_query_len > Q && (pf_mode == 1 || chunky) && (int64_t)num_seqs * Q * nq < INT32_MAX) {
        p.pf_qlen = Q + 1;
        p.pf_tq = pf_tq;
        p.q_lo = 0;
        p.q_hi = 1;
        if (pf_out) *pf_out = PfClass{Q + 1, pf_tq, 2, Q};
        max_query_len = 1;
      }
    }
  }
  // Two 16-row MFMA blocks per wave (int4, one kv head per wave) where a
  // sequence has more than 16 dense rows (query_len x group) to fill: the K
  // and V codes of a step become operands once for 32 rows. Where 16 rows
  // hold a sequence's whole query block, the second block would only add
  // empty rows (measured: qlen 4 x group 4 at 2.9 TB/s with two blocks
  // against 3.9 with one).
  p.rb = 1;
  const int64_t dense_rows = (int64_t)(max_query_len < 1 ? 1 : max_query_len) * G;
  if (mfma && qm == 0 && hs <= 128 && dense_rows > kMfmaRows && env_long("KV4_MFMA_RB", 2) == 2) p.rb = 2;
  const int rmax = mfma ? kMfmaRows * p.rb : kRowsMax;
  p.gh = G < rmax ? G : rmax;
  if (max_query_len <= 1) {
    p.tq = 1;
    p.rows = mfma ? rmax : kv4::host_next_pow2(p.gh);
  } else {
    p.tq = rmax / p.gh;
    if (p.tq < 1) p.tq = 1;
    p.rows = rmax;
  }
  p.n_head_tiles = (G + p.gh - 1) / p.gh;
  // Single-token decode on the matrix cores: one wave serves hpw kv heads
  // (hpw * G <= 16 MFMA rows), sharing its softmax and page walk.
  p.hpw = 1;
  // several heads per wave need the heads of a token row side by side,
  // except at head size 128 where V can be staged per head
  if (mfma && max_query_len <= 1 && qm == 0 && (lay_contig || hs == 128)) {
    long want = env_long("KV4_MFMA_HPW", 0);
    if (want != 1 && want != 2 && want != 4) want = mfma_hpw_max(hs);
    if (mfma_padded_head_size(hs)) want = 1;   // padded rows: one head per wave
    if (want > 2 && (hs == 96 || hs >= 192)) want = 2;   // four heads' V loads would exceed the load counter
    while (want > 1 && (want * G > kMfmaRows || nkv % want != 0)) want >>= 1;
    p.hpw = (int)want;
  }
  p.wpb = kv4::mfma_waves_per_block(p.hpw, qm, hs);
  p.vjh = (p.hpw > 1 && !lay_contig) ? 1 : 0;
  // Single-token decode on the matrix cores, with whole workgroups of kv head
  // groups: stream-K partition of the KV steps over the resident workgroups
  // (no split size; every workgroup gets the same number of steps).
  // (also multi-token decode where every sequence's queries fit one tile)
  p.sk = 0;
  const int mql1 = max_query_len < 1 ? 1 : max_query_len;
  if (mfma && mql1 <= p.tq && p.n_head_tiles == 1 && (nkv / p.hpw) % p.wpb == 0 &&
      env_long("KV4_STREAMK", 1) != 0) {
    p.sk = 1;
    p.sk_quads = nkv / p.hpw / p.wpb;
    const int64_t quads = p.sk_quads;
    const int64_t max_steps = quads * num_seqs * (((int64_t)(max_seq_len < 1 ? 1 : max_seq_len) + 31) / 32);
    // at least kSkMinSteps steps per workgroup, but two workgroups per CU
    // where the LDS holds them
    int64_t cap = std::max<int64_t>(max_steps / kSkMinSteps, std::min<int64_t>(kSkMinGrid, max_steps));
    const long forced = env_long("KV4_SK_GRID", 0);
    if (forced > 0) cap = forced;
    p.sk_pcap = (int)std::max<int64_t>(1, std::min<int64_t>(cap, kSkMaxGrid));
    // int4 head sizes 64 and 96 (two kv heads per wave): one workgroup per
    // CU, each with twice the steps, beats two. Measured with the cache read
    // from HBM (4 rotated copies): Phi-3 shape 32 x 1k 49.9 -> 44.0 us, 64 x
    // 1k 81.2 -> 70.4, 32 x 4k 144 -> 122; Llama-3.2-1B shape 64 x U[1k, 4k]
    // 50.4 -> 48.8, 128 x 84.6 -> 80.6. At head size 128 the Llama-3-8B 32k
    // batch loses 5 % that way and head size 192 22 %, so they keep two.
    p.sk_per_cu = (qm == 0 && hs < 128 && forced <= 0) ? 1 : 0;
  }
  const int mql = max_query_len < 1 ? 1 : max_query_len;
  p.tiles_per_seq = (mql + p.tq - 1) / p.tq;
  const int64_t uniform = (int64_t)num_seqs * p.tiles_per_seq;
  const int64_t packed = num_q_tokens / p.tq + num_seqs;
  if (uniform <= packed) {
    p.packed_tiles = 0;
    p.n_qtiles = uniform;
  } else {
    p.packed_tiles = 1;
    p.n_qtiles = packed;
  }
  const int64_t units = p.n_qtiles * p.n_head_tiles * (nkv / p.hpw);   // waves per split
  if (units > INT32_MAX / 2) return fail(KV4_EUNSUPPORTED, "too many query tiles");
  const int msl = max_seq_len < 1 ? 1 : max_seq_len;
  long split = env_long("KV4_SPLIT_TOKENS", 0);
  if (split <= 0) {
    if (mfma) {
      // A piece of a query tile writes rows x hs fp32 partials whatever its
      // length (16 KB for 32 rows at head size 128), so batches with
      // multi-token tiles aim at half as many, longer pieces (measured on a
      // mixed chunked-prefill batch: 9 splits 11 % faster than 17, 2 splits
      // 15 % slower).
      const int64_t target = max_query_len > 1 ? kTargetUnitsMfma / 2 : kTargetUnitsMfma;
      if (max_query_len > 1 && units >= target) {
        split = msl;                        // prefill tiles already fill the machine
      } else {
        split = (long)((int64_t)msl * units * p.hpw / target);
        if (split < kMinSplit) split = kMinSplit;
        // single-query decode beside the prefill kernel (split-KV where its
        // heads leave no stream-K cut) gets only the CUs the prefill
        // workgroups leave free: fewer, longer pieces there (measured on the
        // mixed Qwen2.5-1.5B batch, 60 decodes over 256-8k contexts beside
        // 4 chunks of 512: splits of 256 tokens 123 us, 512 117, 1024 120,
        // 2048 145)
        if (!cls && p.pf_qlen > 0 && !p.sk && split < 2 * kMinSplit) split = 2 * kMinSplit;
      }
    } else {
      int64_t ns = (kTargetUnitsValu + units - 1) / (units > 0 ? units : 1);
      if (ns < 1) ns = 1;
      split = (msl + ns - 1) / ns;
      if (split < kMinSplit) split = kMinSplit;
    }
  }
  // the launch of the 2 .. Q-query sequences beside the prefill kernel
  // counts every query tile as its own, so it would split finer than the
  // single-kernel plan; at that plan's split size its partials (at most as
  // many rows per split) take no more workspace than that plan's
  if (cls && !p.sk && split < min_split) split = min_split;
  if (mfma) split = (split + 31) / 32 * 32;   // the MFMA kernel walks 32-token steps
  if (split >= msl) split = mfma ? (msl + 31) / 32 * 32 : msl;
  p.split_tokens = (int)split;
  p.num_splits = (int)((msl + split - 1) / split);
  if (p.num_splits > 65535) return fail(KV4_EUNSUPPORTED, "too many KV splits (%d)", p.num_splits);
  if (units * p.num_splits > INT32_MAX / 2) return fail(KV4_EUNSUPPORTED, "too many work units");
  return KV4_OK;
}

// The plan of a call, and with the prefill kernel on the plan of its second
// launch beside it (the sequences with 2 .. Q queries; tile->pf_qlen = 0 where
// there is none), whose key pieces are at least tile_min_split tokens long.
kv4_status make_plan(int qm, int64_t num_q_tokens, int32_t num_seqs, int32_t nq, int32_t nkv, int32_t hs,
              int32_t max_query_len, int32_t max_seq_len, int32_t block_size, const kv4::CacheLayout& lay,
              kv4::AttnPlan& p, kv4::AttnPlan* tile = nullptr, int tile_min_split = 0) {
  PfClass pf{0, 0, 0, 0};
  if (kv4_status e = make_plan_for(qm, num_q_tokens, num_seqs, nq, nkv, hs, max_query_len, max_seq_len, block_size,
                                   lay, p, nullptr, &pf))
    return e;
  if (tile) {
    std::memset(tile, 0, sizeof(*tile));
    if (pf.pf_qlen > 0 && pf.q_hi >= pf.q_lo) {
      kv4::AttnPlan one;
      if (kv4_status e = make_plan_for(qm, num_q_tokens, num_seqs, nq, nkv, hs, max_query_len, max_seq_len,
                                       block_size, lay, one, nullptr, nullptr, true))
        return e;
      return make_plan_for(qm, num_q_tokens, num_seqs, nq, nkv, hs, max_query_len, max_seq_len, block_size, lay,
                           *tile, &pf, nullptr, false, std::max(one.sk ? 0 : one.split_tokens, tile_min_split));
    }
  }
  return KV4_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
  size_t prefix_off, o_off, ml_off, total;
};

WsLayout ws_layout(const kv4::AttnPlan& p, int64_t num_q_tokens, int32_t num_seqs, int32_t nq, int32_t hs) {
  WsLayout w{0, 0, 0, 0};
  if (num_q_tokens == 0) return w;
  size_t off = 0;
  if (p.path == 1) {
    w.prefix_off = 0;
    off = align_up((size_t)(num_seqs + 1) * sizeof(int32_t), 256);
  }
  if (p.sk || p.num_splits > 1) {
    // split-KV: one row per (split, query token, q head); stream-K: one per
    // (range piece, query token of the tile, q head), at most workgroups +
    // quads * sequences pieces
    // (beside the prefill kernel, compact rows: one per (split, sequence,
    // query of the sequence), at most q_hi queries per sequence)
    const size_t qrows = kv4::compact_rows(p) ? (size_t)num_seqs * (size_t)p.q_hi : (size_t)num_q_tokens;
    const size_t rows = p.sk ? ((size_t)p.sk_pcap + (size_t)p.sk_quads * (size_t)num_seqs) * (size_t)p.tq *
                                   (size_t)nq
                             : (size_t)p.num_splits * qrows * (size_t)nq;
    w.o_off = off;
    w.ml_off = align_up(off + rows * (size_t)hs * sizeof(float), 256);
    off = align_up(w.ml_off + rows * 2 * sizeof(float), 256);
  }
  w.total = off;
  return w;
}

// Workspace of a call: its plan's, then (with the prefill kernel) the second
// launch's at the next 256-byte boundary (*tile_off).
size_t plans_ws_bytes(const kv4::AttnPlan& p, const kv4::AttnPlan& tile, int64_t num_q_tokens, int32_t num_seqs,
                      int32_t nq, int32_t hs, size_t* tile_off) {
  size_t total = ws_layout(p, num_q_tokens, num_seqs, nq, hs).total;
  if (tile.pf_qlen > 0) {
    const size_t off = align_up(total, 256);
    if (tile_off) *tile_off = off;
    total = off + ws_layout(tile, num_q_tokens, num_seqs, nq, hs).total;
  }
  return total;
}

kv4_status check_attn_sizes(int64_t num_q_tokens, int32_t num_seqs, int32_t nq, int32_t nkv, int32_t hs,
                     int32_t max_query_len, int32_t max_seq_len) {
  if (num_q_tokens < 0 || num_q_tokens > INT32_MAX)
    return fail(KV4_EINVAL, "num_q_tokens out of range: %lld", (long long)num_q_tokens);
  if (num_seqs < 0) return fail(KV4_EINVAL, "num_seqs must be >= 0, got %d", num_seqs);
  if (num_q_tokens > 0 && num_seqs == 0) return fail(KV4_EINVAL, "num_q_tokens > 0 needs num_seqs >= 1");
  if (nkv < 1 || nkv > 65535) return fail(KV4_EINVAL, "num_kv_heads must be in [1, 65535], got %d", nkv);
  if (nq < 1 || nq % nkv != 0)
    return fail(KV4_EINVAL, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", nq, nkv);
  if (max_query_len < 0 || max_seq_len < 0) return fail(KV4_EINVAL, "max lengths must be >= 0");
  if (hs < 8 || hs > 256 || hs % 8) return fail(KV4_EINVAL, "head_size must be a multiple of 8 in [8, 256]");
  return KV4_OK;
}

kv4_status check_mode(int32_t mode) {
  if (mode != 1 && mode != 2)
    return fail(KV4_EINVAL, "kv_quant_mode must be 1 (int8) or 2 (fp8 e4m3fn), got %d", mode);
  return KV4_OK;
}

kv4_status check_head_pth(int32_t head_size) {
  if (head_size < 8 || head_size > 256 || head_size % 8 != 0)
    return fail(KV4_EINVAL, "head_size must be a multiple of 8 in [8, 256], got %d", head_size);
  return KV4_OK;
}

int64_t code_row_bytes(int qm, int32_t head_size) { return qm ? head_size : head_size / 2; }

// True where every 128-byte line of the K and V code caches that one wave of
// the matrix-core kernel loads is loaded by no other wave: each (sequence, kv
// head) pair has one query tile and one head tile, and the code bytes a wave
// takes from a token row (hpw adjacent heads, or one head) cover whole,
// aligned lines. Those loads then take the non-temporal hint, which keeps the
// streamed codes from displacing lines other waves still need (measured on
// Llama-3-8B-shaped decode: int4 6 % faster, int8 / fp8 11 %). Where lines
// are split between waves (int4 at head sizes 64, 96 and 192, or the
// inline-scale layout) the hint measured 12-28 % slower, with up to 39 % more
// bytes fetched from HBM, so it stays off there.
// The kernels are built with the hint at head size 128 only: int4 with two or
// four adjacent heads per wave, int8 / fp8 (one head of 128 bytes per wave).
bool nt_kernel_built(int qm, int32_t head_size, const kv4::AttnPlan& p) {
  if (p.path == 1 && head_size == 256 && qm == 0) return p.hpw == 1 && !p.vjh && p.rb == 1;   // 128-byte rows
  return p.path == 1 && head_size == 128 && (qm != 0 || (p.hpw >= 2 && !p.vjh && p.rb == 1));
}

bool code_lines_private(int qm, int32_t head_size, const kv4::AttnPlan& p, const kv4::CacheLayout& lay,
                        const void* key_cache, const void* value_cache) {
  if (!nt_kernel_built(qm, head_size, p) || p.n_head_tiles != 1 || p.tiles_per_seq != 1) return false;
  const int64_t cb = code_row_bytes(qm, head_size);
  const int64_t span = (p.hpw > 1 && lay.head == cb) ? p.hpw * cb : cb;   // bytes one wave reads per row
  const bool heads_ok = (p.hpw > 1 && lay.head == cb) ? true : lay.head % 128 == 0;
  return span % 128 == 0 && heads_ok && lay.tok % 128 == 0 && lay.blk % 128 == 0 && aligned(key_cache, 128) &&
         aligned(value_cache, 128);
}

int bs_shift_of(int32_t bs) { return (bs & (bs - 1)) == 0 ? __builtin_ctz((unsigned)bs) : -1; }

// A caller-described layout: positive strides, code strides multiples of the
// kernels' access width (4 bytes int4, 8 bytes int8 / fp8). Rows are not
// checked for overlap (the caller's layout must keep them apart).
kv4_status check_layout(int qm, const kv4::CacheLayout& l) {
  const int64_t A = qm ? 8 : 4;
  if (l.blk <= 0 || l.tok <= 0 || l.head <= 0 || l.sblk <= 0 || l.stok <= 0 || l.shead <= 0)
    return fail(KV4_EINVAL, "layout strides must be positive");
  if (l.blk % A || l.tok % A || l.head % A)
    return fail(KV4_EINVAL, "layout code strides must be multiples of %lld bytes", (long long)A);
  if (l.blk > (INT64_MAX >> 20) || l.sblk > (INT64_MAX >> 22)) return fail(KV4_EINVAL, "layout strides too large");
  return KV4_OK;
}

kv4::CacheLayout to_layout(const kv4_cache_layout* l) {
  kv4::CacheLayout c;
  c.blk = l->block_stride;
  c.tok = l->token_stride;
  c.head = l->head_stride;
  c.sblk = l->scale_block_stride;
  c.stok = l->scale_token_stride;
  c.shead = l->scale_head_stride;
  return c;
}

// Debug check (KV4_CHECK_SLOTS=1): the slot map is copied to the host (the
// call then waits for the stream) and every slot in [0, num_slots) must
// appear at most once -- two tokens in one slot would race.
kv4_status check_unique_slots(const char* what, const int64_t* slot_mapping, int64_t num_tokens, int64_t num_slots,
                       hipStream_t stream) {
  std::vector<int64_t> h((size_t)num_tokens);
  if (kv4_status e = hip_status(hipMemcpyAsync(h.data(), slot_mapping, (size_t)num_tokens * sizeof(int64_t),
                                        hipMemcpyDeviceToHost, stream), what))
    return e;
  if (kv4_status e = hip_status(hipStreamSynchronize(stream), what)) return e;
  std::unordered_map<int64_t, int64_t> first;
  first.reserve((size_t)num_tokens);
  for (int64_t t = 0; t < num_tokens; ++t) {
    const int64_t sl = h[(size_t)t];
    if (sl < 0 || sl >= num_slots) continue;          // skipped by the kernel
    auto ins = first.emplace(sl, t);
    if (!ins.second)
      return fail(KV4_EINVAL, "%s: slot %lld appears at tokens %lld and %lld", what, (long long)sl,
                  (long long)ins.first->second, (long long)t);
  }
  return KV4_OK;
}

kv4_status write_impl(int qm, const char* what, const void* key, const void* value, int64_t key_token_stride,
               int64_t value_token_stride, void* key_cache, void* value_cache, float* k_scale_cache,
               float* v_scale_cache, const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
               int32_t head_size, int32_t b, int32_t block_size, int64_t num_blocks, uint64_t sign_seed,
               void* stream, const kv4::CacheLayout* layout = nullptr) {
  if (num_tokens < 0) return fail(KV4_EINVAL, "num_tokens must be >= 0");
  if (num_kv_heads < 1) return fail(KV4_EINVAL, "num_kv_heads must be >= 1");
  if (block_size < 1 || block_size > 4096) return fail(KV4_EINVAL, "block_size must be in [1, 4096]");
  if (num_blocks < 0) return fail(KV4_EINVAL, "num_blocks must be >= 0");
  if (num_blocks > INT64_MAX / block_size / num_kv_heads / head_size)
    return fail(KV4_EINVAL, "cache too large");
  if (num_tokens == 0) return ok();
  if (num_tokens > INT64_MAX / 2 / num_kv_heads) return fail(KV4_EINVAL, "num_tokens too large");
  const int64_t row = (int64_t)num_kv_heads * head_size;
  if (key_token_stride < row || value_token_stride < row || key_token_stride % 8 || value_token_stride % 8)
    return fail(KV4_EINVAL, "token strides must be >= num_kv_heads*head_size (%lld) and multiples of 8",
                (long long)row);
  if (!key || !value || !key_cache || !value_cache || !k_scale_cache || !v_scale_cache || !slot_mapping)
    return fail(KV4_EINVAL, "null pointer argument");
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16) ||
      !aligned(k_scale_cache, 4) || !aligned(v_scale_cache, 4) || !aligned(slot_mapping, 8))
    return fail(KV4_EINVAL, "misaligned pointer (K/V and caches need 16 bytes)");
  const kv4::CacheLayout lay =
      layout ? *layout : kv4::packed_layout(num_kv_heads, (int)code_row_bytes(qm, head_size), block_size);
  if (kv4_status e = check_layout(qm, lay)) return e;
  if (env_long("KV4_CHECK_SLOTS", 0) != 0) {
    if (kv4_status e = check_unique_slots(what, slot_mapping, num_tokens, num_blocks * block_size,
                                   static_cast<hipStream_t>(stream)))
      return e;
  }
  kv4::WriteArgs a;
  a.key = static_cast<const uint16_t*>(key);
  a.value = static_cast<const uint16_t*>(value);
  a.key_stride = key_token_stride;
  a.value_stride = value_token_stride;
  a.key_cache = static_cast<uint8_t*>(key_cache);
  a.value_cache = static_cast<uint8_t*>(value_cache);
  a.k_scale = k_scale_cache;
  a.v_scale = v_scale_cache;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_slots = num_blocks * block_size;
  a.nkv = num_kv_heads;
  a.hs = head_size;
  a.b = b;
  a.seed = sign_seed;
  a.qm = qm;
  a.bs = block_size;
  a.bs_shift = bs_shift_of(block_size);
  a.lay = lay;
  return hip_status(kv4::launch_write(a, static_cast<hipStream_t>(stream)), what);
}

kv4_status dequant_impl(int qm, const char* what, const void* cache, const float* scale_cache, int64_t num_blocks,
                 const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads, int32_t head_size,
                 int32_t b, int32_t block_size, uint64_t sign_seed, int32_t inverse_rotate, float* out,
                 void* stream, const kv4::CacheLayout* layout = nullptr) {
  if (num_tokens < 0) return fail(KV4_EINVAL, "num_tokens must be >= 0");
  if (num_kv_heads < 1) return fail(KV4_EINVAL, "num_kv_heads must be >= 1");
  if (block_size < 1 || block_size > 4096) return fail(KV4_EINVAL, "block_size must be in [1, 4096]");
  if (num_blocks < 0 || num_blocks > INT64_MAX / block_size / num_kv_heads / head_size)
    return fail(KV4_EINVAL, "num_blocks out of range");
  if (num_tokens == 0) return ok();
  if (!cache || !scale_cache || !slot_mapping || !out) return fail(KV4_EINVAL, "null pointer argument");
  if (!aligned(cache, 16) || !aligned(out, 16) || !aligned(scale_cache, 4) || !aligned(slot_mapping, 8))
    return fail(KV4_EINVAL, "misaligned pointer");
  const kv4::CacheLayout lay =
      layout ? *layout : kv4::packed_layout(num_kv_heads, (int)code_row_bytes(qm, head_size), block_size);
  if (kv4_status e = check_layout(qm, lay)) return e;
  kv4::DequantArgs a;
  a.cache = static_cast<const uint8_t*>(cache);
  a.scale = scale_cache;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_slots = num_blocks * block_size;
  a.nkv = num_kv_heads;
  a.hs = head_size;
  a.b = b;
  a.seed = sign_seed;
  a.inverse_rotate = inverse_rotate ? 1 : 0;
  a.out = out;
  a.qm = qm;
  a.bs = block_size;
  a.bs_shift = bs_shift_of(block_size);
  a.lay = lay;
  return hip_status(kv4::launch_dequant(a, static_cast<hipStream_t>(stream)), what);
}

size_t workspace_impl(int qm, int64_t num_q_tokens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_size, int32_t max_query_len, int32_t max_seq_len,
                      const kv4::CacheLayout* layout = nullptr) {
  if (check_attn_sizes(num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_size, max_query_len,
                       max_seq_len))
    return 0;
  if (layout && check_layout(qm, *layout)) return 0;
  // block_size is not an argument here: size for the larger of the two paths
  size_t need = 0;
  for (int32_t bs : {16, 1}) {
    kv4::AttnPlan p, tile;
    const kv4::CacheLayout lay =
        layout ? *layout : kv4::packed_layout(num_kv_heads, (int)code_row_bytes(qm, head_size), 16);
    if (make_plan(qm, num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_size, max_query_len, max_seq_len,
                  bs, lay, p, &tile))
      return 0;
    const size_t n = plans_ws_bytes(p, tile, num_q_tokens, num_seqs, num_q_heads, head_size, nullptr);
    need = n > need ? n : need;
  }
  g_last_error.clear();
  return need;
}

// A side stream of the current device (default priority, non-blocking) and
// the two events of a fork / join, created once per device and kept for the
// life of the process; mu serializes the fork-launch-join sequences of
// concurrent calls (an event must not be re-recorded between its record and
// the wait on it). nullptr if they cannot be created: the call then runs on
// the caller's stream alone.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};
SideStream* side_stream_on_current_device() {
  static std::mutex mu;
  static std::unordered_map<int, SideStream*> by_dev;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  auto it = by_dev.find(dev);
  if (it != by_dev.end()) return it->second;
  SideStream* s = new SideStream();
  if (hipStreamCreateWithFlags(&s->stream, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&s->fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&s->join, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();   // clear the sticky error: the call goes on without the side stream
    delete s;                  // (handles created before the failure are left to the process exit)
    s = nullptr;
  }
  by_dev[dev] = s;
  return s;
}

kv4_status attention_impl(int qm, const void* query, int64_t query_token_stride, const void* key_cache,
                   const void* value_cache, const float* k_scale_cache, const float* v_scale_cache,
                   int64_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
                   const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                   int64_t num_q_tokens, int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_size, int32_t b, int32_t block_size, uint64_t sign_seed,
                   float softmax_scale, void* out, void* workspace, size_t workspace_bytes, void* stream,
                   const kv4::CacheLayout* layout = nullptr, int32_t window = 0, bool allow_fork = true,
                   bool fit_workspace = false) {
  if (kv4_status e = check_attn_sizes(num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_size, max_query_len,
                               max_seq_len))
    return e;
  if (block_size < 1 || block_size > 4096) return fail(KV4_EINVAL, "block_size must be in [1, 4096]");
  if (num_blocks < 0 || num_blocks > INT32_MAX) return fail(KV4_EINVAL, "num_blocks out of range");
  if (!std::isfinite(softmax_scale)) return fail(KV4_EINVAL, "softmax_scale must be finite");
  if (window < 0) return fail(KV4_EINVAL, "sliding_window must be >= 0 (0 = none), got %d", window);
  if (num_q_tokens == 0) return ok();
  if (num_q_tokens * (int64_t)num_q_heads > INT32_MAX)
    return fail(KV4_EUNSUPPORTED, "num_q_tokens * num_q_heads must be below 2^31");
  if (max_blocks_per_seq < 1) return fail(KV4_EINVAL, "max_blocks_per_seq must be >= 1");
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return fail(KV4_EINVAL, "page table too long");
  if (query_token_stride < (int64_t)num_q_heads * head_size || query_token_stride % 8)
    return fail(KV4_EINVAL, "query_token_stride must be >= num_q_heads*head_size and a multiple of 8");
  if (!query || !key_cache || !value_cache || !k_scale_cache || !v_scale_cache || !block_table || !seq_lens ||
      !query_start_loc || !out)
    return fail(KV4_EINVAL, "null pointer argument");
  if (!aligned(query, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(out, 16) ||
      !aligned(k_scale_cache, 4) || !aligned(v_scale_cache, 4) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || !aligned(query_start_loc, 4))
    return fail(KV4_EINVAL, "misaligned pointer (query, caches and out need 16 bytes)");

  kv4::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  if (num_blocks < 1) return fail(KV4_EINVAL, "num_blocks must be >= 1 when there are query tokens");
  a.lay = layout ? *layout : kv4::packed_layout(num_kv_heads, (int)code_row_bytes(qm, head_size), block_size);
  if (kv4_status e = check_layout(qm, a.lay)) return e;
  kv4::AttnPlan tile_plan;
  if (kv4_status e = make_plan(qm, num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_size, max_query_len,
                       max_seq_len, block_size, a.lay, a.plan, &tile_plan))
    return e;
  size_t tile_off = 0;
  size_t ws_total = plans_ws_bytes(a.plan, tile_plan, num_q_tokens, num_seqs, num_q_heads, head_size, &tile_off);
  // a fixed workspace (the static scratch): the launch of the 2 .. Q-query
  // sequences beside the prefill kernel takes longer key pieces, down to one
  // per tile, until the call fits
  for (int ms = tile_plan.split_tokens * 2; fit_workspace && ws_total > workspace_bytes && tile_plan.pf_qlen > 0 &&
                                            !tile_plan.sk && tile_plan.num_splits > 1 && ms > 0 && ms <= INT32_MAX / 2;
       ms *= 2) {
    if (kv4_status e = make_plan(qm, num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_size, max_query_len,
                                 max_seq_len, block_size, a.lay, a.plan, &tile_plan, ms))
      return e;
    ws_total = plans_ws_bytes(a.plan, tile_plan, num_q_tokens, num_seqs, num_q_heads, head_size, &tile_off);
  }
  // the workspace pointers of one launch's plan, from byte `base` on
  auto place = [&](kv4::AttnArgs& x, size_t base, int32_t*& pfx) {
    const WsLayout w = ws_layout(x.plan, num_q_tokens, num_seqs, num_q_heads, head_size);
    char* wsb = static_cast<char*>(workspace) + base;
    pfx = nullptr;
    if (w.total == 0) return;
    if (x.plan.path == 1) pfx = reinterpret_cast<int32_t*>(wsb + w.prefix_off);
    if (x.plan.sk || x.plan.num_splits > 1) {
      x.ws_o = reinterpret_cast<float*>(wsb + w.o_off);
      x.ws_ml = reinterpret_cast<float*>(wsb + w.ml_off);
    }
  };
  int32_t* prefix = nullptr;
  if (ws_total > 0) {
    if (!workspace || workspace_bytes < ws_total)
      return fail(KV4_EWORKSPACE, "workspace of %zu bytes required, got %zu", ws_total,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(KV4_EINVAL, "workspace must be 16-byte aligned");
    place(a, 0, prefix);
  }
  a.query = static_cast<const uint16_t*>(query);
  a.q_stride = query_token_stride;
  a.key_cache = static_cast<const uint8_t*>(key_cache);
  a.value_cache = static_cast<const uint8_t*>(value_cache);
  a.k_scale = k_scale_cache;
  a.v_scale = v_scale_cache;
  a.num_blocks = num_blocks;
  a.block_table = block_table;
  a.max_blocks = max_blocks_per_seq;
  a.seq_lens = seq_lens;
  a.qsl = query_start_loc;
  a.num_seqs = num_seqs;
  a.num_q_tokens = num_q_tokens;
  a.max_query_len = max_query_len;
  a.max_seq_len = max_seq_len;
  a.nq = num_q_heads;
  a.nkv = num_kv_heads;
  a.hs = head_size;
  a.b = b;
  a.bs = block_size;
  a.seed = sign_seed;
  a.qm = qm;
  // int4: logits scale by softmax_scale / b; the per-token-head modes have no
  // rotation and pass b = 1
  a.scale_log2 = softmax_scale / (float)b * 1.4426950408889634f;
  a.out = static_cast<uint16_t*>(out);
  a.prefix = prefix;
  a.window = window;
  a.code_nt = code_lines_private(qm, head_size, a.plan, a.lay, key_cache, value_cache) ? 1 : 0;
  if (const long f = env_long("KV4_NT", -1); f == 0 || f == 1)
    a.code_nt = (f == 1 && nt_kernel_built(qm, head_size, a.plan)) ? 1 : 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // With a prefill kernel, the other sequences' kernels (decode kernel and
  // merge) run on the device's side stream, forked from and joined back into
  // the caller's stream with events, so they fill the CUs the prefill
  // workgroups leave free instead of queueing behind them. The caller sees
  // one stream-ordered call either way.
  SideStream* side = nullptr;
  std::unique_lock<std::mutex> fork_lock;
  hipStream_t dst = st;
  if (a.plan.pf_qlen > 0 && allow_fork && env_long("KV4_FORK", 1) != 0) {
    side = side_stream_on_current_device();
    if (side) {
      fork_lock = std::unique_lock<std::mutex>(side->mu);
      if (hipEventRecord(side->fork, st) == hipSuccess && hipStreamWaitEvent(side->stream, side->fork, 0) == hipSuccess)
        dst = side->stream;
      else
        side = nullptr;
    }
  }
  // the kernels of one plan (and their merge), on stream `to`
  auto run_plan = [&](kv4::AttnArgs& x, int32_t* pfx, hipStream_t to) -> kv4_status {
    kv4_status r = KV4_OK;
    x.prefix = pfx;
    if (x.plan.path == 1) {
      const int64_t max_units =
          x.plan.n_qtiles * x.plan.n_head_tiles * (num_kv_heads / x.plan.hpw) * x.plan.num_splits;
      r = hip_status(kv4::launch_attn_mfma(x, pfx, max_units, to), "kv4_paged_attention launch");
    } else {
      r = hip_status(kv4::launch_attn_valu(x, to), "kv4_paged_attention launch");
    }
    if (r == KV4_OK && (x.plan.sk || x.plan.num_splits > 1)) {
      // Many rows: one row per lane group (a quarter of the waves at head size
      // 128, each folding its row's partials four loads at a time). Few rows:
      // one row per wave, whose lane groups split the partials, so that more
      // waves share the latency-bound work (measured: 2048 rows at head size 64
      // 7 % faster per wave; 20k-25k rows 3-9 % faster per group).
      const int64_t ng = 64 / kv4::host_next_pow2(head_size / 8);
      // the merge's rows: beside the prefill kernel (compact rows) only those
      // of the sequences this launch serves, q_hi queries per sequence
      const int64_t mrows =
          (kv4::compact_rows(x.plan) ? (int64_t)num_seqs * x.plan.q_hi : num_q_tokens) * num_q_heads;
      x.reduce_rows = (mrows / ng >= kReduceRowsMinWaves) ? 1 : 0;
      if (const long f = env_long("KV4_REDUCE_ROWS", -1); f == 0 || f == 1) x.reduce_rows = (int)f;
      r = hip_status(kv4::launch_attn_reduce(x, to), "kv4_paged_attention merge launch");
    }
    return r;
  };
  kv4_status rc = run_plan(a, prefix, dst);
  if (rc == KV4_OK && tile_plan.pf_qlen > 0) {
    // the sequences with 2 .. Q queries: their own launch, with its own
    // workspace region
    kv4::AttnArgs t = a;
    t.plan = tile_plan;
    t.plan.wg_cap = kTileLaunchWgs;
    t.code_nt = code_lines_private(qm, head_size, t.plan, t.lay, key_cache, value_cache) ? 1 : 0;
    t.ws_o = nullptr;
    t.ws_ml = nullptr;
    int32_t* tpfx = nullptr;
    place(t, tile_off, tpfx);
    rc = run_plan(t, tpfx, dst);
  }
  // The prefill kernel is enqueued after the decode kernel: the short,
  // memory-bound decode workgroups then spread over every CU first, and each
  // CU takes its prefill workgroup (which fills its register file) as its
  // decode work drains, instead of the decode kernel squeezing onto the few
  // CUs the prefill workgroups leave.
  if (rc == KV4_OK && a.plan.pf_qlen > 0)
    rc = hip_status(kv4::launch_attn_prefill(a, st), "kv4_paged_attention prefill launch");
  if (side) {
    // join: the caller's stream waits for the side stream's work (also after
    // a failed launch, so nothing of this call is left unordered)
    if (hipEventRecord(side->join, side->stream) != hipSuccess || hipStreamWaitEvent(st, side->join, 0) != hipSuccess)
      if (rc == KV4_OK) rc = fail(KV4_EHIP, "kv4_paged_attention: joining the side stream failed");
  }
  return rc == KV4_OK ? ok() : rc;
}

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr with the error set if
// the lookup fails.
void* scratch_on_current_device() {
  static std::mutex mu;
  static std::unordered_map<int, void*> by_dev;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    fail(KV4_EHIP, "kv4_paged_attention_noalloc: no current HIP device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  auto it = by_dev.find(dev);
  if (it != by_dev.end()) return it->second;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    fail(KV4_EHIP, "kv4_paged_attention_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
         hipGetErrorString(e));
    return nullptr;
  }
  by_dev.emplace(dev, ptr);
  return ptr;
}

}  // namespace

extern "C" {

const char* kv4_last_error(void) { return g_last_error.c_str(); }

kv4_status kv4_paged_attention_noalloc(const void* query, int64_t query_token_stride, const void* key_cache,
                                       const void* value_cache, const float* k_scale_cache,
                                       const float* v_scale_cache, int64_t num_blocks, const int32_t* block_table,
                                       int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                       const int32_t* query_start_loc, int32_t num_seqs, int64_t num_q_tokens,
                                       int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_size, int32_t b, int32_t block_size,
                                       uint64_t sign_seed, float softmax_scale, void* out, void* stream) {
  if (kv4_status e = check_head(head_size, b)) return e;
  void* ws = scratch_on_current_device();
  if (!ws) return KV4_EHIP;
  const kv4_status st =
      attention_impl(0, query, query_token_stride, key_cache, value_cache, k_scale_cache, v_scale_cache,
                     num_blocks, block_table, max_blocks_per_seq, seq_lens, query_start_loc, num_seqs, num_q_tokens,
                     max_query_len, max_seq_len, num_q_heads, num_kv_heads, head_size, b, block_size, sign_seed,
                     softmax_scale, out, ws, (size_t)KV4_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0,
                     /*allow_fork=*/false, /*fit_workspace=*/true);
  if (st == KV4_EWORKSPACE) {
    const std::string why = g_last_error;
    return fail(KV4_EWORKSPACE,
                "kv4_paged_attention_noalloc: %s; the static scratch holds %zu bytes -- call "
                "kv4_paged_attention with a caller workspace for this batch",
                why.c_str(), (size_t)KV4_NOALLOC_SCRATCH_BYTES);
  }
  return st;
}

kv4_status kv4_debug_flags(uint32_t* flags, int32_t clear) {
  if (!flags) return fail(KV4_EINVAL, "flags must not be null");
  *flags = 0;
#ifdef KV4_DEBUG
  if (kv4_status e = hip_status(hipDeviceSynchronize(), "kv4_debug_flags: device synchronize")) return e;
  const bool c = clear != 0;
  *flags = kv4::debug_flags_write(c) | kv4::debug_flags_mfma(c) | kv4::debug_flags_prefill(c) |
           kv4::debug_flags_valu(c);
  return ok();
#else
  (void)clear;
  return fail(KV4_EUNSUPPORTED, "kv4_debug_flags: this library is built without KV4_DEBUG");
#endif
}

kv4_status kv4_stream_read(const void* buffer, int64_t bytes, uint32_t* sink, int32_t grid, void* stream) {
  if (bytes < 0 || bytes % 16) return fail(KV4_EINVAL, "bytes must be a non-negative multiple of 16");
  if (grid < 1 || grid > 65536) return fail(KV4_EINVAL, "grid must be in [1, 65536], got %d", grid);
  if (bytes == 0) return ok();
  if (!buffer || !sink) return fail(KV4_EINVAL, "null pointer argument");
  if (!aligned(buffer, 16) || !aligned(sink, 4)) return fail(KV4_EINVAL, "misaligned pointer");
  return hip_status(kv4::launch_stream_read(buffer, bytes, sink, grid, static_cast<hipStream_t>(stream)),
                    "kv4_stream_read");
}

kv4_status kv4_rht_write(const void* key, const void* value, int64_t key_token_stride,
                  int64_t value_token_stride, void* key_cache, void* value_cache,
                  float* k_scale_cache, float* v_scale_cache, const int64_t* slot_mapping,
                  int64_t num_tokens, int32_t num_kv_heads, int32_t head_size, int32_t b,
                  int32_t block_size, int64_t num_blocks, uint64_t sign_seed, void* stream) {
  if (kv4_status e = check_head(head_size, b)) return e;
  return write_impl(0, "kv4_rht_write", key, value, key_token_stride, value_token_stride, key_cache,
                    value_cache, k_scale_cache, v_scale_cache, slot_mapping, num_tokens, num_kv_heads,
                    head_size, b, block_size, num_blocks, sign_seed, stream);
}

kv4_status kv4_pth_write(int32_t kv_quant_mode, const void* key, const void* value, int64_t key_token_stride,
                  int64_t value_token_stride, void* key_cache, void* value_cache, float* k_scale_cache,
                  float* v_scale_cache, const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                  int32_t head_size, int32_t block_size, int64_t num_blocks, void* stream) {
  if (kv4_status e = check_mode(kv_quant_mode)) return e;
  if (kv4_status e = check_head_pth(head_size)) return e;
  return write_impl(kv_quant_mode, "kv4_pth_write", key, value, key_token_stride, value_token_stride,
                    key_cache, value_cache, k_scale_cache, v_scale_cache, slot_mapping, num_tokens,
                    num_kv_heads, head_size, 0, block_size, num_blocks, 0, stream);
}


size_t kv4_paged_attention_workspace_size(int64_t num_q_tokens, int32_t num_seqs, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_size, int32_t max_query_len,
                                          int32_t max_seq_len) {
  return workspace_impl(0, num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_size, max_query_len,
                        max_seq_len);
}

size_t kv4_pth_attention_workspace_size(int32_t kv_quant_mode, int64_t num_q_tokens, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                                        int32_t max_query_len, int32_t max_seq_len) {
  if (check_mode(kv_quant_mode)) return 0;
  return workspace_impl(kv_quant_mode, num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_size,
                        max_query_len, max_seq_len);
}


kv4_status kv4_paged_attention(const void* query, int64_t query_token_stride, const void* key_cache,
                        const void* value_cache, const float* k_scale_cache, const float* v_scale_cache,
                        int64_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
                        const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                        int64_t num_q_tokens, int32_t max_query_len, int32_t max_seq_len,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size, int32_t b,
                        int32_t block_size, uint64_t sign_seed, float softmax_scale, void* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (kv4_status e = check_head(head_size, b)) return e;
  return attention_impl(0, query, query_token_stride, key_cache, value_cache, k_scale_cache, v_scale_cache,
                        num_blocks, block_table, max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                        num_q_tokens, max_query_len, max_seq_len, num_q_heads, num_kv_heads, head_size, b,
                        block_size, sign_seed, softmax_scale, out, workspace, workspace_bytes, stream);
}

kv4_status kv4_pth_attention(int32_t kv_quant_mode, const void* query, int64_t query_token_stride,
                      const void* key_cache, const void* value_cache, const float* k_scale_cache,
                      const float* v_scale_cache, int64_t num_blocks, const int32_t* block_table,
                      int32_t max_blocks_per_seq, const int32_t* seq_lens, const int32_t* query_start_loc,
                      int32_t num_seqs, int64_t num_q_tokens, int32_t max_query_len, int32_t max_seq_len,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                      float softmax_scale, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (kv4_status e = check_mode(kv_quant_mode)) return e;
  if (kv4_status e = check_head_pth(head_size)) return e;
  return attention_impl(kv_quant_mode, query, query_token_stride, key_cache, value_cache, k_scale_cache,
                        v_scale_cache, num_blocks, block_table, max_blocks_per_seq, seq_lens, query_start_loc,
                        num_seqs, num_q_tokens, max_query_len, max_seq_len, num_q_heads, num_kv_heads, head_size,
                        1, block_size, 0, softmax_scale, out, workspace, workspace_bytes, stream);
}


kv4_status kv4_dequant(const void* cache, const float* scale_cache, int64_t num_blocks, const int64_t* slot_mapping,
                int64_t num_tokens, int32_t num_kv_heads, int32_t head_size, int32_t b, int32_t block_size,
                uint64_t sign_seed, int32_t inverse_rotate, float* out, void* stream) {
  if (kv4_status e = check_head(head_size, b)) return e;
  return dequant_impl(0, "kv4_dequant", cache, scale_cache, num_blocks, slot_mapping, num_tokens, num_kv_heads,
                      head_size, b, block_size, sign_seed, inverse_rotate, out, stream);
}

kv4_status kv4_pth_dequant(int32_t kv_quant_mode, const void* cache, const float* scale_cache, int64_t num_blocks,
                    const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads, int32_t head_size,
                    int32_t block_size, float* out, void* stream) {
  if (kv4_status e = check_mode(kv_quant_mode)) return e;
  if (kv4_status e = check_head_pth(head_size)) return e;
  return dequant_impl(kv_quant_mode, "kv4_pth_dequant", cache, scale_cache, num_blocks, slot_mapping, num_tokens,
                      num_kv_heads, head_size, 0, block_size, 0, 0, out, stream);
}


kv4_status kv4_cache_layout_packed(int32_t kv_quant_mode, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                            kv4_cache_layout* layout) {
  if (kv_quant_mode < 0 || kv_quant_mode > 2) return fail(KV4_EINVAL, "kv_quant_mode must be 0, 1 or 2");
  if (num_kv_heads < 1 || head_size < 8 || head_size % 8 || block_size < 1 || !layout)
    return fail(KV4_EINVAL, "invalid sizes or null layout");
  const kv4::CacheLayout l = kv4::packed_layout(num_kv_heads, (int)code_row_bytes(kv_quant_mode, head_size),
                                                block_size);
  *layout = kv4_cache_layout{l.blk, l.tok, l.head, l.sblk, l.stok, l.shead};
  return ok();
}

kv4_status kv4_cache_layout_inline(int32_t kv_quant_mode, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                            kv4_cache_layout* layout, int64_t* block_bytes, int64_t* value_offset,
                            int64_t* scale_offset) {
  if (kv_quant_mode < 0 || kv_quant_mode > 2) return fail(KV4_EINVAL, "kv_quant_mode must be 0, 1 or 2");
  if (num_kv_heads < 1 || head_size < 8 || head_size % 8 || block_size < 1 || block_size > 4096 || !layout)
    return fail(KV4_EINVAL, "invalid sizes or null layout");
  const int64_t c = code_row_bytes(kv_quant_mode, head_size);
  const int64_t pitch = (c + 4 + 15) / 16 * 16;               // codes, fp32 scale, zero padding
  const int64_t half = (int64_t)block_size * num_kv_heads * pitch;
  *layout = kv4_cache_layout{2 * half, num_kv_heads * pitch, pitch, 2 * half / 4, num_kv_heads * pitch / 4,
                             pitch / 4};
  if (block_bytes) *block_bytes = 2 * half;
  if (value_offset) *value_offset = half;
  if (scale_offset) *scale_offset = c;
  return ok();
}

namespace {
kv4_status check_any_mode(int32_t mode, int32_t head_size, int32_t& b) {
  if (mode == 0) return check_head(head_size, b);
  if (kv4_status e = check_mode(mode)) return e;
  return check_head_pth(head_size);
}
}  // namespace

kv4_status kv4_write_layout(int32_t kv_quant_mode, const void* key, const void* value, int64_t key_token_stride,
                     int64_t value_token_stride, void* key_cache, void* value_cache, float* k_scale_cache,
                     float* v_scale_cache, const kv4_cache_layout* layout, const int64_t* slot_mapping,
                     int64_t num_tokens, int32_t num_kv_heads, int32_t head_size, int32_t b, int32_t block_size,
                     int64_t num_blocks, uint64_t sign_seed, void* stream) {
  if (kv4_status e = check_any_mode(kv_quant_mode, head_size, b)) return e;
  if (!layout) return fail(KV4_EINVAL, "null layout");
  const kv4::CacheLayout l = to_layout(layout);
  return write_impl(kv_quant_mode, "kv4_write_layout", key, value, key_token_stride, value_token_stride,
                    key_cache, value_cache, k_scale_cache, v_scale_cache, slot_mapping, num_tokens, num_kv_heads,
                    head_size, kv_quant_mode ? 1 : b, block_size, num_blocks, kv_quant_mode ? 0 : sign_seed,
                    stream, &l);
}

size_t kv4_attention_layout_workspace_size(int32_t kv_quant_mode, const kv4_cache_layout* layout,
                                           int64_t num_q_tokens, int32_t num_seqs, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_size, int32_t max_query_len,
                                           int32_t max_seq_len) {
  if (kv_quant_mode != 0 && check_mode(kv_quant_mode)) return 0;
  if (!layout) {
    fail(KV4_EINVAL, "null layout");
    return 0;
  }
  const kv4::CacheLayout l = to_layout(layout);
  return workspace_impl(kv_quant_mode, num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_size, max_query_len,
                        max_seq_len, &l);
}

kv4_status kv4_attention_layout(int32_t kv_quant_mode, const void* query, int64_t query_token_stride,
                         const void* key_cache, const void* value_cache, const float* k_scale_cache,
                         const float* v_scale_cache, const kv4_cache_layout* layout, int64_t num_blocks,
                         const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                         const int32_t* query_start_loc, int32_t num_seqs, int64_t num_q_tokens,
                         int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_size, int32_t b, int32_t block_size, uint64_t sign_seed,
                         int32_t sliding_window, float softmax_scale, void* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (kv4_status e = check_any_mode(kv_quant_mode, head_size, b)) return e;
  if (!layout) return fail(KV4_EINVAL, "null layout");
  const kv4::CacheLayout l = to_layout(layout);
  return attention_impl(kv_quant_mode, query, query_token_stride, key_cache, value_cache, k_scale_cache,
                        v_scale_cache, num_blocks, block_table, max_blocks_per_seq, seq_lens, query_start_loc,
                        num_seqs, num_q_tokens, max_query_len, max_seq_len, num_q_heads, num_kv_heads, head_size,
                        kv_quant_mode ? 1 : b, block_size, kv_quant_mode ? 0 : sign_seed, softmax_scale, out,
                        workspace, workspace_bytes, stream, &l, sliding_window);
}

kv4_status kv4_dequant_layout(int32_t kv_quant_mode, const void* cache, const float* scale_cache,
                       const kv4_cache_layout* layout, int64_t num_blocks, const int64_t* slot_mapping,
                       int64_t num_tokens, int32_t num_kv_heads, int32_t head_size, int32_t b, int32_t block_size,
                       uint64_t sign_seed, int32_t inverse_rotate, float* out, void* stream) {
  if (kv4_status e = check_any_mode(kv_quant_mode, head_size, b)) return e;
  if (!layout) return fail(KV4_EINVAL, "null layout");
  const kv4::CacheLayout l = to_layout(layout);
  return dequant_impl(kv_quant_mode, "kv4_dequant_layout", cache, scale_cache, num_blocks, slot_mapping,
                      num_tokens, num_kv_heads, head_size, kv_quant_mode ? 1 : b, block_size,
                      kv_quant_mode ? 0 : sign_seed, kv_quant_mode ? 0 : inverse_rotate, out, stream, &l);
}

}  // extern "C"
