// Host side of the centroid-masked sparse LM head: argument validation,
// derived tables, workspace layout and the stream-ordered sequence of kernels
// for each entry point of include/ce.h.
//
// The head follows Gemma4MTPMaskedEmbedder of the vLLM compare view "[Spec
// Decode] Add Gemma4 MTP speculative decoding with centroids masking" (diff of
// gemma4_mtp.py).  Its token_ordering buffer, read as slot -> token id and
// viewed as [num_centroids, vocab_size_per_centroid], becomes token_of_slot
// plus cluster offsets (equal clusters when no offsets are given).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <functional>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/ce.h"
#include "ce_internal.h"

static_assert(CE_STATIC_SCRATCH_BYTES == ce::kStaticScratchBytes,
              "the header's static scratch size is the library's");

struct ce_head {
  int32_t d = 0, V = 0, Nc = 0, max_B = 0, max_K = 0, dtype = 0, slab = CE_SLAB_NATIVE;
  int32_t proj = CE_PROJ_AUTO;
  unsigned long long* stats = nullptr;   // device: [cmax bits, ..., repaired rows, recomputed rows]
  const void* C = nullptr;
  const void* E = nullptr;
  std::vector<int32_t> offsets;       // [Nc+1]
  std::vector<int32_t> tos;           // [V]
  // Equal tile counts per cluster (tpc > 0): every 64-slot tile of every
  // cluster, (index in cluster << 13) | cluster, zero-padded past the
  // cluster's end.  Otherwise (tpc == 0, `tiles` empty) the contiguous
  // tiling: tile t holds slots [64t, 64t+64) and tcl their clusters.
  std::vector<uint32_t> tiles;
  int tpc = 0;                        // tiles per cluster if all clusters hold as many, else 0
  long long n_tiles = 0;
  std::vector<int32_t> ttok;          // [n_tiles][64] token id of each tile slot, -1 past the end
  std::vector<uint16_t> tcl;          // tpc == 0: [n_tiles][64] cluster of each slot
  // tiles_top[K] = the most tiles the rows of K clusters touch (a bound on
  // a row's tile segments): each cluster's tiles, summed over the K largest
  std::vector<long long> tiles_top;
  bool prepared = false;
  ce::Tables tables{};
};

struct ce_graph {
  hipGraphExec_t exec = nullptr;
};

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_probe_start = nullptr;
thread_local hipEvent_t g_probe_stop = nullptr;

ce_status fail(ce_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

ce_status fail_hip(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return CE_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t elem_bytes(int dtype) { return dtype == CE_BF16 ? 2 : 4; }

// Workspace regions of one pass (at most ce::kPassRows rows).
struct Layout {
  size_t scores = 0, topk = 0, cl_sel = 0, best = 0, amax = 0, tm_keys = 0, tm_heads = 0, tm_rank = 0,
         crec = 0, hnorm = 0, total = 0;
  bool has_rank = false;
  bool cert = false;
  int tm_segcap = 0;
};

// ce_top_tokens on a bf16 head takes the certified matrix-core argmax
// with CE_PROJ_MFMA, and with CE_PROJ_AUTO where it measured faster than
// the float64 dot: hidden sizes from 512, where each slot's chain is long,
// and ragged heads, whose tiles carry many rows (B=64: skewed head, d=512,
// gather 21.7 against 32.9 µs; wide head, d=1024, call 83.8 against 106.7;
// sweep head, d=256, 23.4 against 20.8 the other way).
bool cert_head(const ce_head* h) {
  // the records carry token ids in 25 bits
  if (h->dtype != CE_BF16 || h->proj == CE_PROJ_EXACT || h->V > (1 << 25)) return false;
  return h->proj == CE_PROJ_MFMA || h->d >= 512 || h->tpc == 0;
}

// CE_PROJ_AUTO takes the MFMA projection for a pass of at least this many
// multiply-adds (B Nc d).  The exact projection costs in proportion to them;
// the certified top-K adds a few microseconds whatever their number (its
// band recomputation included).  The sweep head (d = 256, Nc = 2048) stays
// exact up to B = 64 (2^25), where MFMA measured 1-2 µs slower; the skewed
// head (d = 512, Nc = 2048) at B = 64 (2^26) takes it: 46.3 -> 42.1 µs per
// call, with no other benchmark row changed.
constexpr long long kMfmaMinMacs = 1ll << 26;

// The two forms of the fused top-m (logits, or log-probabilities).
bool top_m_op(int op) { return op == CE_OP_TOP_M || op == CE_OP_TOP_M_LOG_SOFTMAX; }

Layout make_layout(const ce_head* h, int B, int K, int op, bool allow_cert = true) {
  Layout L;
  const size_t nb = (size_t)std::min(B, ce::kPassRows);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  if (op == CE_OP_SCORE) {
    L.total = 0;
    return L;
  }
  L.scores = take(nb * h->Nc * sizeof(float));
  L.topk = take(nb * (size_t)K * sizeof(int32_t));
  L.cl_sel = take(((size_t)h->Nc + 63) / 64 * ce::kPassRows * sizeof(unsigned long long));
  L.best = take(ce::kPassRows * sizeof(unsigned long long));
  L.amax = take(ce::kArgWords * sizeof(unsigned long long));
  if (op == CE_OP_TOP_TOKENS && allow_cert && cert_head(h)) {
    // one 16-byte record per (row, tile): padded tiling, in the order of
    // the row's selected clusters (their ranks from the top-K); contiguous,
    // by tile
    L.cert = true;
    L.hnorm = take(ce::kPassRows * sizeof(float));
    if (h->tpc > 0) {
      L.crec = take(nb * (size_t)K * h->tpc * 16);
      L.tm_rank = take(nb * (size_t)h->Nc * sizeof(int16_t));
      L.has_rank = true;
    } else {
      L.crec = take(nb * (size_t)h->n_tiles * 16);
    }
  }
  if (top_m_op(op)) {
    L.tm_segcap = (int)std::max<long long>(h->tiles_top[K], 1);
    L.tm_keys = take(nb * (size_t)L.tm_segcap * ce::kTileTokens * sizeof(unsigned long long));
    L.tm_heads = take(nb * (size_t)L.tm_segcap * sizeof(unsigned long long));
    if (h->tpc > 0) {   // equal clusters: fixed segment places
      L.tm_rank = take(nb * (size_t)h->Nc * sizeof(int16_t));
      L.has_rank = true;
    }
  }
  L.total = off;
  return L;
}

// Offsets of the device tables inside the persistent buffer.
struct PersistLayout {
  size_t stats, offsets, tos, tiles, ttok, tcl, et, escale, enorm, ct, total;
};

PersistLayout persist_layout(const ce_head* h) {
  PersistLayout p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  p.stats = take(ce::kStatsWords * sizeof(unsigned long long));
  p.offsets = take(((size_t)h->Nc + 1) * sizeof(int32_t));
  p.tos = take((size_t)h->V * sizeof(int32_t));
  p.tiles = take(std::max<size_t>(h->tiles.size(), 1) * sizeof(uint32_t));
  p.ttok = take(std::max<size_t>(h->ttok.size(), 1) * sizeof(int32_t));
  p.tcl = h->tcl.empty() ? 0 : take(h->tcl.size() * sizeof(uint16_t));
  const size_t tile_bytes = (size_t)ce::kTileTokens * h->d * elem_bytes(h->dtype);
  const size_t slab_tile = h->slab == CE_SLAB_FP8_E4M3 ? (size_t)ce::kTileTokens * h->d : tile_bytes;
  const size_t n_tiles = (size_t)h->n_tiles;
  p.et = take(n_tiles * slab_tile);
  p.escale = h->slab == CE_SLAB_FP8_E4M3 ? take(n_tiles * ce::kTileTokens * sizeof(float)) : 0;
  p.enorm = h->dtype == CE_BF16 ? take(n_tiles * ce::kTileTokens * sizeof(float)) : 0;
  p.ct = take((((size_t)h->Nc + ce::kTileTokens - 1) / ce::kTileTokens) * tile_bytes);
  p.total = off;
  return p;
}

ce_status check_call(const ce_head* h, const void* in, int B, int K, bool needs_k) {
  if (!h) return fail(CE_ERR_NULL_POINTER, "head is NULL");
  if (!h->prepared) return fail(CE_ERR_NOT_PREPARED, "ce_head_prepare has not been called");
  if (B < 0 || B > h->max_B) return fail(CE_ERR_BAD_SHAPE, "B must lie in [0, max_B]");
  if (needs_k && (K < 1 || K > h->max_K)) return fail(CE_ERR_BAD_SHAPE, "K must lie in [1, max_K]");
  if (B > 0 && !in) return fail(CE_ERR_NULL_POINTER, "input pointer is NULL");
  return CE_SUCCESS;
}

ce::PassArgs base_args(const ce_head* h, int K) {
  ce::PassArgs a;
  std::memset(&a, 0, sizeof(a));
  a.dtype = h->dtype;
  a.d = h->d;
  a.V = h->V;
  a.Nc = h->Nc;
  a.K = K;
  a.C = h->C;
  a.E = h->E;
  a.t = h->tables;
  return a;
}

void bind_workspace(ce::PassArgs& a, const Layout& L, char* ws) {
  a.S = reinterpret_cast<float*>(ws + L.scores);
  a.ldS = a.Nc;
  a.topk = reinterpret_cast<int32_t*>(ws + L.topk);
  a.ldK = a.K;
  a.cl_sel = reinterpret_cast<unsigned long long*>(ws + L.cl_sel);
  a.best = reinterpret_cast<unsigned long long*>(ws + L.best);
  a.amax = reinterpret_cast<unsigned long long*>(ws + L.amax);
  a.tm_keys = reinterpret_cast<unsigned long long*>(ws + L.tm_keys);
  a.tm_heads = reinterpret_cast<unsigned long long*>(ws + L.tm_heads);
  a.tm_segcap = L.tm_segcap;
  a.tm_rank = L.has_rank ? reinterpret_cast<int16_t*>(ws + L.tm_rank) : nullptr;
  a.ldR = a.Nc;
  a.cert = L.cert;
  a.crec = L.cert ? ws + L.crec : nullptr;
  a.hnorm = L.cert ? reinterpret_cast<float*>(ws + L.hnorm) : nullptr;
}

// The draft step's extra operands (ce_draft_step).
struct DraftArgs {
  const void* norm_w;
  float eps;
  void* h_out;
  const void* emb_table;
  int emb_dim;
  float normalizer;
  void* emb_out;
};

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

ce_status check_draft(const ce_head* h, const void* x, int B, const DraftArgs& dr) {
  if (!(dr.eps > 0.0f) || !std::isfinite(dr.eps)) return fail(CE_ERR_BAD_SHAPE, "eps must be finite and > 0");
  if (dr.emb_table) {
    if (dr.emb_dim < 1 || ((size_t)dr.emb_dim * elem_bytes(h->dtype)) % 16)
      return fail(CE_ERR_BAD_SHAPE, "emb_dim must be > 0 with 16-byte rows");
    if (!std::isfinite(dr.normalizer)) return fail(CE_ERR_BAD_SHAPE, "normalizer must be finite");
  }
  if (B == 0) return CE_SUCCESS;
  if (!dr.norm_w || !dr.h_out || (dr.emb_table && !dr.emb_out))
    return fail(CE_ERR_NULL_POINTER, "norm_weight, h_out and (with a table) emb_out are required");
  if (!aligned(dr.norm_w, 16) || !aligned(dr.h_out, 16) ||
      (dr.emb_table && (!aligned(dr.emb_table, 16) || !aligned(dr.emb_out, 16))))
    return fail(CE_ERR_MISALIGNED, "norm_weight, h_out, emb_table and emb_out need 16-byte alignment");
  const size_t rows = (size_t)B * h->d * elem_bytes(h->dtype);
  if (overlaps(x, rows, dr.h_out, rows)) return fail(CE_ERR_UNSUPPORTED, "x and h_out overlap");
  return CE_SUCCESS;
}

// The shared sequence of ce_top_tokens, ce_masked_logits, ce_top_m and
// ce_draft_step, in passes of at most kPassRows rows.
ce_status run_sparse(ce_head* h, int op, const void* hin, int B, int K, void* out,
                     int32_t* topk_ids, void* ws, size_t ws_bytes, hipStream_t stream,
                     int m = 0, float* out2 = nullptr, const DraftArgs* draft = nullptr,
                     bool dry = false, bool allow_cert = true) {
  ce_status st = check_call(h, hin, B, K, true);
  if (st != CE_SUCCESS) return st;
  if (op == CE_OP_DRAFT_STEP) {
    st = check_draft(h, hin, B, *draft);
    if (st != CE_SUCCESS) return st;
  }
  if (B > 0 && (!out || (top_m_op(op) && !out2)))
    return fail(CE_ERR_NULL_POINTER, "output pointer is NULL");
  if (top_m_op(op)) {
    if (m < 1 || m > ce::kMaxTopM) return fail(CE_ERR_BAD_SHAPE, "m must lie in [1, CE_MAX_TOP_M]");
    if (h->tiles_top[K] + (long long)m * ce::kTileTokens > ce::kTopMLdsWords)
      return fail(CE_ERR_UNSUPPORTED, "the K largest clusters hold too many tiles for the top-m merge");
  }
  if (B == 0) return CE_SUCCESS;
  if (!ws) return fail(CE_ERR_NULL_POINTER, "workspace is NULL");
  if (!aligned(hin, 16) || !aligned(out, op == CE_OP_MASKED_LOGITS ? 16 : 4) || !aligned(ws, 256) ||
      (topk_ids && !aligned(topk_ids, 4)) || (out2 && !aligned(out2, 4)))
    return fail(CE_ERR_MISALIGNED, "h and logits need 16-byte, ws 256-byte alignment");
  const Layout L = make_layout(h, B, K, op, allow_cert);
  if (ws_bytes < L.total) return fail(CE_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than ce_workspace_bytes");
  if (dry) return CE_SUCCESS;   // arguments checked, nothing enqueued

  hipEvent_t pstart = g_probe_start, pstop = g_probe_stop;
  g_probe_start = g_probe_stop = nullptr;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (pstart && hipStreamIsCapturing(stream, &cap) == hipSuccess && cap != hipStreamCaptureStatusNone)
    pstart = pstop = nullptr;

  const size_t in_row = (size_t)h->d * elem_bytes(h->dtype);
  for (int b0 = 0; b0 < B; b0 += ce::kPassRows) {
    const int nb = std::min(ce::kPassRows, B - b0);
    ce::PassArgs a = base_args(h, K);
    a.B = nb;
    a.h = static_cast<const char*>(hin) + (size_t)b0 * in_row;
    a.approx = op != CE_OP_DRAFT_STEP &&
               (h->proj == CE_PROJ_MFMA ||
                (h->proj == CE_PROJ_AUTO && (long long)nb * h->Nc * h->d >= kMfmaMinMacs));
    bind_workspace(a, L, static_cast<char*>(ws));
    if (topk_ids) {
      a.topk = topk_ids + (size_t)b0 * K;
      a.ldK = K;
    }
    if (op == CE_OP_TOP_TOKENS || op == CE_OP_DRAFT_STEP) {
      a.tokens = static_cast<int32_t*>(out) + b0;
    } else if (top_m_op(op)) {
      a.m = m;
      a.tm_log_softmax = op == CE_OP_TOP_M_LOG_SOFTMAX;
      a.tm_cap = L.tm_segcap * ce::kTileTokens;
      a.tm_tokens = static_cast<int32_t*>(out) + (size_t)b0 * m;
      a.tm_logits = out2 + (size_t)b0 * m;
    } else {
      a.logits = static_cast<float*>(out) + (size_t)b0 * h->V;
      a.fill = a.logits;
    }
    if (b0 == 0) {
      a.probe_start = pstart;
      a.probe_stop = pstop;
    }
    const int mode = op == CE_OP_MASKED_LOGITS ? ce::kMasked : top_m_op(op) ? ce::kTopM : ce::kArgmax;
    void* h_out = nullptr;
    if (op == CE_OP_DRAFT_STEP) {
      // scores reads the rows before the norm and writes the normalised ones
      h_out = static_cast<char*>(draft->h_out) + (size_t)b0 * in_row;
      a.norm_w = draft->norm_w;
      a.norm_eps = draft->eps;
      a.h_out = h_out;
      if (draft->emb_table) {
        a.emb_table = draft->emb_table;
        a.emb_dim = draft->emb_dim;
        a.emb_normalizer = draft->normalizer;
        a.emb_out = static_cast<char*>(draft->emb_out) +
                    (size_t)b0 * draft->emb_dim * elem_bytes(h->dtype);
      }
    }
    hipError_t e = ce::launch_scores(a, stream);
    if (h_out) {
      a.h = h_out;   // the rest of the pass works on the normalised rows
      a.norm_w = nullptr;
    }
    if (e == hipSuccess) e = ce::launch_topk(a, ce::kTopkMark, stream);
    if (e == hipSuccess) e = ce::launch_gather(a, mode, stream);
    if (e == hipSuccess && mode == ce::kArgmax) e = ce::launch_finalize(a, stream);
    if (e == hipSuccess && mode == ce::kTopM) e = ce::launch_topm_merge(a, stream);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
  }
  return CE_SUCCESS;
}

}  // namespace

extern "C" {

ce_status ce_head_create(const ce_head_desc* desc, ce_head_t* out) {
  if (!desc || !out) return fail(CE_ERR_NULL_POINTER, "desc or out is NULL");
  *out = nullptr;
  if (!desc->centroids || !desc->emb_ordered || !desc->token_of_slot)
    return fail(CE_ERR_NULL_POINTER, "centroids, emb_ordered and token_of_slot are required");
  if (desc->dtype != CE_F32 && desc->dtype != CE_BF16) return fail(CE_ERR_BAD_DTYPE, "dtype must be CE_F32 or CE_BF16");
  if (desc->slab_format != CE_SLAB_NATIVE && desc->slab_format != CE_SLAB_FP8_E4M3)
    return fail(CE_ERR_BAD_DTYPE, "slab_format must be CE_SLAB_NATIVE or CE_SLAB_FP8_E4M3");
  if (desc->slab_format == CE_SLAB_FP8_E4M3 && desc->dtype != CE_BF16)
    return fail(CE_ERR_BAD_DTYPE, "FP8 slabs are quantised from bf16 heads only");
  if (desc->projection < CE_PROJ_AUTO || desc->projection > CE_PROJ_MFMA)
    return fail(CE_ERR_BAD_DTYPE, "projection must be CE_PROJ_AUTO, CE_PROJ_EXACT or CE_PROJ_MFMA");
  if (desc->projection == CE_PROJ_MFMA && desc->dtype != CE_BF16)
    return fail(CE_ERR_BAD_DTYPE, "the MFMA projection takes bf16 heads only");
  const int d = desc->d, V = desc->V, Nc = desc->Nc;
  if (d < 64 || d > ce::kMaxD || d % 64) return fail(CE_ERR_BAD_SHAPE, "d must be a multiple of 64 in [64, 8192]");
  if (V < 1) return fail(CE_ERR_BAD_SHAPE, "V must be >= 1");
  if (Nc < 1 || Nc > ce::kMaxNc) return fail(CE_ERR_BAD_SHAPE, "Nc must lie in [1, 8192]");
  if (desc->max_B < 1) return fail(CE_ERR_BAD_SHAPE, "max_B must be >= 1");
  if (desc->max_K < 1 || desc->max_K > Nc) return fail(CE_ERR_BAD_SHAPE, "max_K must lie in [1, Nc]");
  if (!aligned(desc->centroids, 16) || !aligned(desc->emb_ordered, 16))
    return fail(CE_ERR_MISALIGNED, "centroids and emb_ordered need 16-byte alignment");

  ce_head* h = new (std::nothrow) ce_head;
  if (!h) return fail(CE_ERR_UNSUPPORTED, "out of host memory");
  h->d = d;
  h->V = V;
  h->Nc = Nc;
  h->max_B = desc->max_B;
  h->max_K = desc->max_K;
  h->dtype = desc->dtype;
  h->slab = desc->slab_format;
  h->proj = desc->dtype == CE_BF16 ? desc->projection : CE_PROJ_EXACT;
  h->C = desc->centroids;
  h->E = desc->emb_ordered;
  try {
    h->offsets.resize((size_t)Nc + 1);
    if (desc->cluster_offsets) {
      std::memcpy(h->offsets.data(), desc->cluster_offsets, h->offsets.size() * sizeof(int32_t));
      if (h->offsets[0] != 0 || h->offsets[Nc] != V) {
        delete h;
        return fail(CE_ERR_BAD_LAYOUT, "offsets must start at 0 and end at V");
      }
      for (int c = 0; c < Nc; ++c)
        if (h->offsets[c + 1] < h->offsets[c]) {
          delete h;
          return fail(CE_ERR_BAD_LAYOUT, "offsets must be nondecreasing");
        }
    } else {
      if (V % Nc) {
        delete h;
        return fail(CE_ERR_BAD_LAYOUT, "equal clusters need V % Nc == 0");
      }
      for (int c = 0; c <= Nc; ++c) h->offsets[c] = (int32_t)((long long)c * (V / Nc));
    }
    h->tos.assign(desc->token_of_slot, desc->token_of_slot + V);
    std::vector<char> seen((size_t)V, 0);
    for (int j = 0; j < V; ++j) {
      const int32_t t = h->tos[j];
      if (t < 0 || t >= V || seen[t]) {
        delete h;
        return fail(CE_ERR_BAD_LAYOUT, "token_of_slot must be a permutation of 0..V-1");
      }
      seen[t] = 1;
    }
    std::vector<long long> ntiles((size_t)Nc);
    for (int c = 0; c < Nc; ++c) {
      const long long size = h->offsets[c + 1] - h->offsets[c];
      ntiles[c] = (size + ce::kTileTokens - 1) / ce::kTileTokens;
      if (ntiles[c] > ce::kMaxTilesPerCluster) {
        delete h;
        return fail(CE_ERR_UNSUPPORTED, "a cluster holds more than 2^19 * 64 tokens");
      }
    }
    h->tpc = (int)ntiles[0];
    for (int c = 1; c < Nc; ++c)
      if (ntiles[c] != ntiles[0]) h->tpc = 0;
    if (h->tpc > 0) {
      for (int c = 0; c < Nc; ++c)
        for (long long q = 0; q < ntiles[c]; ++q) {
          h->tiles.push_back(((uint32_t)q << ce::kTileShift) | (uint32_t)c);
          for (int l = 0; l < ce::kTileTokens; ++l) {
            const long long j = h->offsets[c] + q * ce::kTileTokens + l;
            h->ttok.push_back(j < h->offsets[c + 1] ? h->tos[j] : -1);
          }
        }
      h->n_tiles = (long long)h->tiles.size();
    } else {
      // contiguous tiling: no padding, so a tile may hold several clusters
      // and a cluster's first and last tiles may be shared
      h->n_tiles = ((long long)V + ce::kTileTokens - 1) / ce::kTileTokens;
      h->ttok.assign((size_t)h->n_tiles * ce::kTileTokens, -1);
      h->tcl.assign((size_t)h->n_tiles * ce::kTileTokens, (uint16_t)ce::kNoCluster);
      for (int c = 0; c < Nc; ++c) {
        const long long lo = h->offsets[c], hi = h->offsets[c + 1];
        for (long long j = lo; j < hi; ++j) {
          h->ttok[(size_t)j] = h->tos[(size_t)j];
          h->tcl[(size_t)j] = (uint16_t)c;
        }
        ntiles[c] = hi > lo ? (hi - 1) / ce::kTileTokens - lo / ce::kTileTokens + 1 : 0;
      }
    }
    std::sort(ntiles.begin(), ntiles.end(), std::greater<long long>());
    h->tiles_top.assign((size_t)Nc + 1, 0);
    for (int k = 0; k < Nc; ++k) h->tiles_top[k + 1] = h->tiles_top[k] + ntiles[k];
  } catch (const std::bad_alloc&) {
    delete h;
    return fail(CE_ERR_UNSUPPORTED, "out of host memory");
  }
  *out = h;
  return CE_SUCCESS;
}

ce_status ce_head_destroy(ce_head_t head) {
  delete head;
  return CE_SUCCESS;
}

ce_status ce_head_persistent_bytes(ce_head_t head, size_t* bytes) {
  if (!head || !bytes) return fail(CE_ERR_NULL_POINTER, "head or bytes is NULL");
  *bytes = persist_layout(head).total;
  return CE_SUCCESS;
}

ce_status ce_head_prepare(ce_head_t head, void* persistent, size_t bytes, hipStream_t stream) {
  if (!head || !persistent) return fail(CE_ERR_NULL_POINTER, "head or persistent buffer is NULL");
  if (!aligned(persistent, 256)) return fail(CE_ERR_MISALIGNED, "persistent buffer needs 256-byte alignment");
  const PersistLayout p = persist_layout(head);
  if (bytes < p.total) return fail(CE_ERR_WORKSPACE_TOO_SMALL, "persistent buffer too small");
  char* base = static_cast<char*>(persistent);
  struct Copy {
    size_t at;
    const std::vector<int32_t>* v;
  } copies[] = {{p.offsets, &head->offsets}, {p.tos, &head->tos}, {p.ttok, &head->ttok}};
  for (const Copy& c : copies) {
    hipError_t e = hipMemcpyAsync(base + c.at, c.v->data(), c.v->size() * sizeof(int32_t),
                                  hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync");
  }
  if (!head->tiles.empty()) {
    hipError_t e = hipMemcpyAsync(base + p.tiles, head->tiles.data(), head->tiles.size() * sizeof(uint32_t),
                                  hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync");
  }
  if (!head->tcl.empty()) {
    hipError_t e = hipMemcpyAsync(base + p.tcl, head->tcl.data(), head->tcl.size() * sizeof(uint16_t),
                                  hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync");
  }
  // the tile list of the padded tiling; the contiguous one packs rows in order
  const uint32_t* tiles_dev =
      head->tiles.empty() ? nullptr : reinterpret_cast<const uint32_t*>(base + p.tiles);
  hipError_t e = hipMemsetAsync(base + p.stats, 0, ce::kStatsWords * sizeof(unsigned long long), stream);
  if (e != hipSuccess) return fail_hip(e, "hipMemsetAsync");
  e = ce::launch_cnorm_max(head->C, head->dtype, head->Nc, head->d,
                           reinterpret_cast<unsigned long long*>(base + p.stats), stream);
  if (e != hipSuccess) return fail_hip(e, "norm kernel launch");
  e = head->slab == CE_SLAB_FP8_E4M3
          ? ce::launch_pack_fp8(head->E, head->d, (long)head->n_tiles, tiles_dev,
                                reinterpret_cast<const int32_t*>(base + p.offsets), head->V,
                                base + p.et, reinterpret_cast<float*>(base + p.escale), stream)
          : ce::launch_pack(head->E, head->dtype, head->d, (long)head->n_tiles, tiles_dev,
                            reinterpret_cast<const int32_t*>(base + p.offsets), head->V,
                            base + p.et, stream);
  if (e == hipSuccess)
    e = ce::launch_pack(head->C, head->dtype, head->d,
                        ((long)head->Nc + ce::kTileTokens - 1) / ce::kTileTokens, nullptr, nullptr,
                        head->Nc, base + p.ct, stream);
  if (e != hipSuccess) return fail_hip(e, "pack kernel launch");
  if (head->dtype == CE_BF16) {
    e = ce::launch_slot_norms(base + p.et, head->slab == CE_SLAB_FP8_E4M3 ? 1 : 0,
                              reinterpret_cast<const float*>(base + p.escale), (long)head->n_tiles,
                              head->d, reinterpret_cast<float*>(base + p.enorm), stream);
    if (e != hipSuccess) return fail_hip(e, "norm kernel launch");
  }
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
  head->tables.offsets = reinterpret_cast<const int32_t*>(base + p.offsets);
  head->tables.tos = reinterpret_cast<const int32_t*>(base + p.tos);
  head->tables.n_tiles = (int)head->n_tiles;
  head->tables.tpc = head->tpc;
  head->tables.ttok = reinterpret_cast<const int32_t*>(base + p.ttok);
  head->tables.tcl = head->tcl.empty() ? nullptr : reinterpret_cast<const uint16_t*>(base + p.tcl);
  head->tables.ET = base + p.et;
  head->tables.slab = head->slab == CE_SLAB_FP8_E4M3 ? 1 : 0;
  head->tables.escale = head->slab == CE_SLAB_FP8_E4M3 ? reinterpret_cast<const float*>(base + p.escale)
                                                        : nullptr;
  head->tables.CT = base + p.ct;
  head->tables.enorm = head->dtype == CE_BF16 ? reinterpret_cast<const float*>(base + p.enorm) : nullptr;
  head->stats = reinterpret_cast<unsigned long long*>(base + p.stats);
  head->tables.stats = head->stats;
  head->prepared = true;
  return CE_SUCCESS;
}

ce_status ce_workspace_bytes(ce_head_t head, int32_t B, int32_t K, int32_t op, size_t* bytes) {
  if (!head || !bytes) return fail(CE_ERR_NULL_POINTER, "head or bytes is NULL");
  if (op < CE_OP_SCORE || op > CE_OP_TOP_M_LOG_SOFTMAX) return fail(CE_ERR_UNSUPPORTED, "unknown op");
  if (B < 0 || B > head->max_B) return fail(CE_ERR_BAD_SHAPE, "B must lie in [0, max_B]");
  if (op == CE_OP_TOPK) {
    *bytes = 0;
    return CE_SUCCESS;
  }
  if (op != CE_OP_SCORE && (K < 1 || K > head->max_K)) return fail(CE_ERR_BAD_SHAPE, "K must lie in [1, max_K]");
  *bytes = make_layout(head, B, op == CE_OP_SCORE ? 1 : K, op).total;
  return CE_SUCCESS;
}

}  // extern "C"

namespace {

ce_status score_impl(ce_head_t head, const void* h, int32_t B, float* scores, hipStream_t stream,
                     bool dry) {
  ce_status st = check_call(head, h, B, 1, false);
  if (st != CE_SUCCESS) return st;
  if (B == 0) return CE_SUCCESS;
  if (!scores) return fail(CE_ERR_NULL_POINTER, "scores is NULL");
  if (!aligned(h, 16) || !aligned(scores, 4)) return fail(CE_ERR_MISALIGNED, "h needs 16-byte alignment");
  if (dry) return CE_SUCCESS;
  for (int b0 = 0; b0 < B; b0 += ce::kPassRows) {
    ce::PassArgs a = base_args(head, 1);
    a.B = std::min(ce::kPassRows, B - b0);
    a.h = static_cast<const char*>(h) + (size_t)b0 * (size_t)head->d * elem_bytes(head->dtype);
    a.S = scores + (size_t)b0 * head->Nc;
    a.ldS = head->Nc;
    hipError_t e = ce::launch_scores(a, stream);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
  }
  return CE_SUCCESS;
}

ce_status topk_impl(ce_head_t head, const float* scores, int32_t B, int32_t K, int32_t* topk_ids,
                    hipStream_t stream, bool dry) {
  ce_status st = check_call(head, scores, B, K, true);
  if (st != CE_SUCCESS) return st;
  if (B == 0) return CE_SUCCESS;
  if (!topk_ids) return fail(CE_ERR_NULL_POINTER, "topk_ids is NULL");
  if (!aligned(scores, 4) || !aligned(topk_ids, 4)) return fail(CE_ERR_MISALIGNED, "scores and ids need 4-byte alignment");
  if (dry) return CE_SUCCESS;
  for (int b0 = 0; b0 < B; b0 += ce::kPassRows) {
    ce::PassArgs a = base_args(head, K);
    a.B = std::min(ce::kPassRows, B - b0);
    a.S = const_cast<float*>(scores) + (size_t)b0 * head->Nc;
    a.ldS = head->Nc;
    a.topk = topk_ids + (size_t)b0 * K;
    a.ldK = K;
    hipError_t e = ce::launch_topk(a, ce::kTopkOnly, stream);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
  }
  return CE_SUCCESS;
}

}  // namespace

extern "C" {

ce_status ce_score_centroids(ce_head_t head, const void* h, int32_t B, float* scores,
                             hipStream_t stream) {
  return score_impl(head, h, B, scores, stream, false);
}

ce_status ce_topk(ce_head_t head, const float* scores, int32_t B, int32_t K, int32_t* topk_ids,
                  hipStream_t stream) {
  return topk_impl(head, scores, B, K, topk_ids, stream, false);
}

ce_status ce_top_tokens(ce_head_t head, const void* h, int32_t B, int32_t K, int32_t* tokens,
                        int32_t* topk_ids_or_null, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_sparse(head, CE_OP_TOP_TOKENS, h, B, K, tokens, topk_ids_or_null, ws, ws_bytes, stream);
}

ce_status ce_top_tokens_static(ce_head_t head, const void* h, int32_t B, int32_t K, int32_t* tokens,
                               int32_t* topk_ids_or_null, hipStream_t stream) {
  ce_status st = check_call(head, h, B, K, true);
  if (st != CE_SUCCESS) return st;
  // the certified argmax's records where they fit, else the float64 dot
  // (the same tokens)
  const bool cert = make_layout(head, B, K, CE_OP_TOP_TOKENS).total <= ce::kStaticScratchBytes;
  const size_t need = make_layout(head, B, K, CE_OP_TOP_TOKENS, cert).total;
  if (need > ce::kStaticScratchBytes)
    return fail(CE_ERR_UNSUPPORTED, "this call needs " + std::to_string(need) +
                                        " bytes of workspace; the static scratch holds " +
                                        std::to_string(ce::kStaticScratchBytes) +
                                        " (use ce_top_tokens with a workspace)");
  if (B == 0) return CE_SUCCESS;
  void* ws = nullptr;
  const hipError_t e = ce::static_scratch(&ws);
  if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
  return run_sparse(head, CE_OP_TOP_TOKENS, h, B, K, tokens, topk_ids_or_null, ws,
                    ce::kStaticScratchBytes, stream, 0, nullptr, nullptr, false, cert);
}

ce_status ce_masked_logits(ce_head_t head, const void* h, int32_t B, int32_t K, float* logits,
                           int32_t* topk_ids_or_null, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_sparse(head, CE_OP_MASKED_LOGITS, h, B, K, logits, topk_ids_or_null, ws, ws_bytes, stream);
}

ce_status ce_top_m(ce_head_t head, const void* h, int32_t B, int32_t K, int32_t m, int32_t* tokens,
                   float* logits, int32_t* topk_ids_or_null, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_sparse(head, CE_OP_TOP_M, h, B, K, tokens, topk_ids_or_null, ws, ws_bytes, stream, m, logits);
}

ce_status ce_top_m_log_softmax(ce_head_t head, const void* h, int32_t B, int32_t K, int32_t m,
                               int32_t* tokens, float* logprobs, int32_t* topk_ids_or_null, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  return run_sparse(head, CE_OP_TOP_M_LOG_SOFTMAX, h, B, K, tokens, topk_ids_or_null, ws, ws_bytes,
                    stream, m, logprobs);
}

ce_status ce_draft_step(ce_head_t head, const void* x, const void* norm_weight, float eps,
                        int32_t B, int32_t K, void* h_out, int32_t* tokens,
                        const void* emb_table, int32_t emb_dim, float normalizer,
                        void* emb_out, int32_t* topk_ids_or_null, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  const DraftArgs dr{norm_weight, eps, h_out, emb_table, emb_dim, normalizer, emb_out};
  return run_sparse(head, CE_OP_DRAFT_STEP, x, B, K, tokens, topk_ids_or_null, ws, ws_bytes,
                    stream, 0, nullptr, &dr);
}

}  // extern "C"

namespace {

// Enqueue one described call, or with `dry` only check its arguments (no
// HIP call is made then).
ce_status enqueue_call(ce_head_t head, const ce_call& c, hipStream_t stream, bool dry) {
  switch (c.op) {
    case CE_OP_SCORE:
      return score_impl(head, c.in, c.B, static_cast<float*>(c.out), stream, dry);
    case CE_OP_TOPK:
      return topk_impl(head, static_cast<const float*>(c.in), c.B, c.K,
                       static_cast<int32_t*>(c.out), stream, dry);
    case CE_OP_TOP_TOKENS:
    case CE_OP_MASKED_LOGITS:
      return run_sparse(head, c.op, c.in, c.B, c.K, c.out, c.topk_ids, c.ws, c.ws_bytes, stream, 0,
                        nullptr, nullptr, dry);
    case CE_OP_TOP_M:
    case CE_OP_TOP_M_LOG_SOFTMAX:
      return run_sparse(head, c.op, c.in, c.B, c.K, c.out, c.topk_ids, c.ws, c.ws_bytes, stream,
                        c.m, c.out_logits, nullptr, dry);
    case CE_OP_DRAFT_STEP: {
      const DraftArgs dr{c.norm_weight, c.eps, c.h_out, c.emb_table, c.emb_dim, c.normalizer,
                         c.emb_out};
      return run_sparse(head, c.op, c.in, c.B, c.K, c.out, c.topk_ids, c.ws, c.ws_bytes, stream, 0,
                        nullptr, &dr, dry);
    }
    default:
      return fail(CE_ERR_UNSUPPORTED, "unknown op");
  }
}

ce_status capture(ce_head_t head, const ce_call& c, hipStream_t stream, ce_graph_t* graph) {
  if (c.op < CE_OP_SCORE || c.op > CE_OP_TOP_M_LOG_SOFTMAX) return fail(CE_ERR_UNSUPPORTED, "unknown op");
  if (!stream) return fail(CE_ERR_UNSUPPORTED, "capture needs a non-null stream");
  // check the call before capturing, so that a bad call leaves no capture
  ce_status st = enqueue_call(head, c, stream, true);
  if (st != CE_SUCCESS) return st;
  hipError_t e = hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return fail_hip(e, "hipStreamBeginCapture");
  st = enqueue_call(head, c, stream, false);
  const std::string call_error = g_last_error;
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(stream, &g);
  if (st != CE_SUCCESS) {
    if (g) (void)hipGraphDestroy(g);
    return fail(st, call_error);
  }
  if (e != hipSuccess) return fail_hip(e, "hipStreamEndCapture");
  ce_graph* out_g = new (std::nothrow) ce_graph;
  if (!out_g) {
    (void)hipGraphDestroy(g);
    return fail(CE_ERR_UNSUPPORTED, "out of host memory");
  }
  e = hipGraphInstantiate(&out_g->exec, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e != hipSuccess) {
    delete out_g;
    return fail_hip(e, "hipGraphInstantiate");
  }
  *graph = out_g;
  return CE_SUCCESS;
}

}  // namespace

extern "C" {

ce_status ce_graph_capture(ce_head_t head, int32_t op, const void* h, int32_t B, int32_t K, void* out,
                           int32_t* topk_ids_or_null, void* ws, size_t ws_bytes, hipStream_t stream,
                           ce_graph_t* graph) {
  if (!graph) return fail(CE_ERR_NULL_POINTER, "graph is NULL");
  *graph = nullptr;
  if (op != CE_OP_SCORE && op != CE_OP_TOPK && op != CE_OP_TOP_TOKENS && op != CE_OP_MASKED_LOGITS)
    return fail(CE_ERR_UNSUPPORTED,
                "ce_graph_capture takes CE_OP_SCORE, TOPK, TOP_TOKENS and MASKED_LOGITS; "
                "use ce_graph_capture_call for the others");
  ce_call c;
  std::memset(&c, 0, sizeof(c));
  c.op = op;
  c.in = h;
  c.B = B;
  c.K = K;
  c.out = out;
  c.topk_ids = topk_ids_or_null;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  return capture(head, c, stream, graph);
}

ce_status ce_graph_capture_call(ce_head_t head, const ce_call* call, hipStream_t stream,
                                ce_graph_t* graph) {
  if (!graph || !call) return fail(CE_ERR_NULL_POINTER, "call or graph is NULL");
  *graph = nullptr;
  return capture(head, *call, stream, graph);
}

ce_status ce_graph_launch(ce_graph_t graph, hipStream_t stream) {
  if (!graph || !graph->exec) return fail(CE_ERR_NULL_POINTER, "graph is NULL");
  hipError_t e = hipGraphLaunch(graph->exec, stream);
  if (e != hipSuccess) return fail_hip(e, "hipGraphLaunch");
  return CE_SUCCESS;
}

ce_status ce_graph_destroy(ce_graph_t graph) {
  if (!graph) return CE_SUCCESS;
  if (graph->exec) (void)hipGraphExecDestroy(graph->exec);
  delete graph;
  return CE_SUCCESS;
}

ce_status ce_probe_gather_events(hipEvent_t start, hipEvent_t stop) {
  if (!start || !stop) return fail(CE_ERR_NULL_POINTER, "events are NULL");
  g_probe_start = start;
  g_probe_stop = stop;
  return CE_SUCCESS;
}

ce_status ce_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink) return fail(CE_ERR_NULL_POINTER, "buf or sink is NULL");
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (bytes & 15u) != 0)
    return fail(CE_ERR_MISALIGNED, "buf and bytes must be multiples of 16");
  const hipError_t e = ce::launch_stream_read(buf, bytes, sink, stream);
  if (e != hipSuccess) return fail(CE_ERR_HIP, hipGetErrorString(e));
  return CE_SUCCESS;
}

ce_status ce_head_repair_counts(ce_head_t head, uint64_t counts[2]) {
  if (!head || !counts) return fail(CE_ERR_NULL_POINTER, "head or counts is NULL");
  if (!head->prepared) return fail(CE_ERR_NOT_PREPARED, "ce_head_prepare has not been called");
  unsigned long long c[2] = {0, 0};
  const hipError_t e = hipMemcpy(c, head->stats + ce::kStatsCounters, sizeof(c), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail_hip(e, "hipMemcpy");
  counts[0] = c[0];
  counts[1] = c[1];
  return CE_SUCCESS;
}

ce_status ce_probe_approx_scores(ce_head_t head, const void* h, int32_t B, float* scores,
                                 hipStream_t stream) {
  ce_status st = check_call(head, h, B, 1, false);
  if (st != CE_SUCCESS) return st;
  if (head->dtype != CE_BF16) return fail(CE_ERR_BAD_DTYPE, "the MFMA projection takes bf16 heads only");
  if (B == 0) return CE_SUCCESS;
  if (!scores) return fail(CE_ERR_NULL_POINTER, "scores is NULL");
  if (!aligned(h, 16) || !aligned(scores, 4)) return fail(CE_ERR_MISALIGNED, "h needs 16-byte alignment");
  for (int b0 = 0; b0 < B; b0 += ce::kPassRows) {
    ce::PassArgs a = base_args(head, 1);
    a.B = std::min(ce::kPassRows, B - b0);
    a.h = static_cast<const char*>(h) + (size_t)b0 * (size_t)head->d * elem_bytes(head->dtype);
    a.S = scores + (size_t)b0 * head->Nc;
    a.ldS = head->Nc;
    a.approx = true;
    hipError_t e = ce::launch_scores(a, stream);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
  }
  return CE_SUCCESS;
}

const char* ce_status_string(ce_status status) {
  switch (status) {
    case CE_SUCCESS: return "CE_SUCCESS";
    case CE_ERR_NULL_POINTER: return "CE_ERR_NULL_POINTER";
    case CE_ERR_BAD_SHAPE: return "CE_ERR_BAD_SHAPE";
    case CE_ERR_BAD_DTYPE: return "CE_ERR_BAD_DTYPE";
    case CE_ERR_MISALIGNED: return "CE_ERR_MISALIGNED";
    case CE_ERR_BAD_LAYOUT: return "CE_ERR_BAD_LAYOUT";
    case CE_ERR_WORKSPACE_TOO_SMALL: return "CE_ERR_WORKSPACE_TOO_SMALL";
    case CE_ERR_NOT_PREPARED: return "CE_ERR_NOT_PREPARED";
    case CE_ERR_HIP: return "CE_ERR_HIP";
    case CE_ERR_UNSUPPORTED: return "CE_ERR_UNSUPPORTED";
  }
  return "CE_UNKNOWN_STATUS";
}

const char* ce_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
