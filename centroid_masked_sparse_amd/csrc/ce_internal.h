// Internal interface between the host library (ce_host.cpp) and the HIP
// kernels (ce_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace ce {

constexpr int kPassRows = 64;     // rows per internal pass: row sets are 64-bit masks
constexpr int kTileTokens = 64;   // candidate tokens per gather work item (one per lane)
constexpr int kMaxNc = 8192;      // centroid id fits the low 13 bits of a work item
constexpr int kTileShift = 13;     // tile word: (tile index in cluster << 13) | cluster
constexpr int kMaxTilesPerCluster = 1 << (32 - kTileShift);
constexpr int kMaxD = 8192;
constexpr int kNoCluster = 0xFFFF;  // slot past the vocabulary in a tile of the contiguous tiling
// The repair counters sit a 128-byte line after the centroid norm that every
// certified top-K row reads first: device-scope atomics on them then never
// touch the norm's line.
constexpr int kStatsCounters = 16;
constexpr int kStatsWords = 32;     // the stats region, 256 bytes

// Device tables uploaded at prepare time.
struct Tables {
  const int32_t* offsets;      // [Nc+1] cluster c owns slots [offsets[c], offsets[c+1])
  const int32_t* tos;          // [V] token id of each slot
  // Two tilings.  When every cluster holds the same number of 64-slot tiles
  // (tpc > 0), each tile belongs to one cluster, zero-padded past its end:
  // tile t is tile t % tpc of cluster t / tpc.  Otherwise tile t holds slots
  // [64t, 64t+64) whatever their clusters, and tcl names each slot's.
  int n_tiles;
  int tpc;                     // tiles per cluster when every cluster holds as many, else 0
  const int32_t* ttok;         // [n_tiles][64] token id of each tile slot, -1 past the end
  const uint16_t* tcl;         // tpc == 0: [n_tiles][64] cluster of each slot, kNoCluster past V
  const void* ET;              // packed embeddings: [n_tiles][d/vec][64] 16-byte vectors
  int slab;                    // 0: the head's dtype; 1: E4M3 codes (16 per vector)
  const float* escale;         // E4M3 slabs: [n_tiles][64] row scales
  const float* enorm;          // [n_tiles][64] |e| of each slot (times its scale), rounded up
  const void* CT;              // packed centroids:  [ceil(Nc/64)][d/vec][64]
  // [0] the largest centroid row norm (bits of a double, rounded up);
  // [kStatsCounters] rows whose top-K band was recomputed in canonical
  // keys, [kStatsCounters + 1] rows recomputed whole (both counted since
  // prepare, atomically)
  unsigned long long* stats;
};

// Argmax slots: a row's packed (ordered logit, ~token) maxima sit in
// kArgSlots words kArgSlotStride words (16 KiB) apart, rows kArgRowStride
// words (256 B) apart inside a slot's block; a gather wave max-es into the
// slot of its index mod kArgSlots and the finalize takes the largest.
// Device-scope atomics on one address serialise, and on neighbouring words
// share a memory channel; the spread slots keep thousands of them per call
// from queueing on one.
constexpr int kArgSlots = 8;
constexpr int kArgRowStride = 32;
constexpr int kArgSlotStride = kPassRows * kArgRowStride;
constexpr size_t kArgWords = (size_t)(kPassRows - 1) * kArgRowStride +
                             (size_t)(kArgSlots - 1) * kArgSlotStride + 1;

enum GatherMode { kArgmax = 0, kMasked = 1, kTopM = 2 };
constexpr int kMaxTopM = 32;        // m of the fused top-m
// 64-bit LDS words of the top-m merge (under 64 KiB with its static part):
// the row's segment heads, then up to m * 64 candidate keys
constexpr int kTopMLdsWords = (65536 - 256) / 8;
// What the top-K kernel writes besides the ids: nothing, or the rows'
// selection words (and, given `best`, cleared argmax slots).
enum TopkMode { kTopkOnly = 1, kTopkMark = 2 };

// Everything one pass (at most kPassRows rows) needs.
struct PassArgs {
  int dtype;              // CE_F32 or CE_BF16
  int d, V, Nc, K;
  int B;                  // rows in this pass, 1..kPassRows
  const void* C;          // [Nc][d]
  const void* E;          // [V][d] ordered layout
  Tables t;
  const void* h;          // [B][d] rows of this pass
  bool approx;            // bf16 MFMA projection + certified top-K (else canonical scores)
  bool cert;              // argmax by matrix-core dots + certified finalize (tile grid only)
  void* crec;             // cert: 16-byte bound records per (row, tile)
  float* hnorm;           // cert: [kPassRows] each row's |h|, rounded up
  // workspace regions
  float* S;               // [B][ldS] centroid scores
  int ldS;
  int32_t* topk;          // [B][ldK] selected centroids
  int ldK;
  unsigned long long* cl_sel;   // [ceil(Nc/64)][kPassRows] bit i of word (w, b): row b selected 64w+i
  unsigned long long* best;     // [kPassRows] top-m counters (segments << 32 | keys)
  unsigned long long* amax;     // [kArgWords] argmax slots (see kArgSlots)
  // fused top-m: per row, a packed count (segments << 32 | keys) in `best`,
  // the tiles' local top-m keys and each tile segment's head key
  int m;
  unsigned long long* tm_keys;   // [B][tm_cap]
  unsigned long long* tm_heads;  // [B][tm_segcap]
  int tm_cap, tm_segcap;
  int16_t* tm_rank;       // equal clusters: [B][ldR] output position of each selected
  int ldR;                // centroid (top-K writes it, the gather's fixed segments read it)
  int32_t* tm_tokens;     // [B][m]
  float* tm_logits;       // [B][m] logits, or log-probabilities with tm_log_softmax
  bool tm_log_softmax;    // top-m: log-softmax over the row's candidates
  // fused draft step: h holds the rows before the final RMSNorm when norm_w
  // is set; the scores kernel writes the normalised rows to h_out (which the
  // gather then reads), and the finalize kernel writes the chosen tokens'
  // scaled embeddings when emb_table is set
  const void* norm_w;     // [d] or null
  float norm_eps;
  void* h_out;            // [B][d]
  const void* emb_table;  // [V][emb_dim] or null
  int emb_dim;
  float emb_normalizer;
  void* emb_out;          // [B][emb_dim]
  // outputs
  int32_t* tokens;        // [B]
  float* logits;          // [B][V] forward output
  float* fill;            // [B][V] rows the scores kernel's extra waves fill with -inf, or null
  // measurement hook (HIP extended launch around the gather kernel)
  hipEvent_t probe_start;
  hipEvent_t probe_stop;
};

// Pack rows of W into 64-row tiles [t][v][lane]: tile t of the cluster
// tile list `tiles` ((index in cluster << 13) | cluster), or rows
// [64t, 64t+64) of nrows_total without one (see ce_kernels.hip).
hipError_t launch_pack(const void* W, int dtype, int d, long n_tiles, const uint32_t* tiles,
                       const int32_t* offsets, int nrows_total, void* out, hipStream_t s);
// Quantise bf16 rows to E4M3 with row scales and pack them the same way.
hipError_t launch_pack_fp8(const void* W, int d, long n_tiles, const uint32_t* tiles,
                           const int32_t* offsets, int nrows_total, void* out, float* scale,
                           hipStream_t s);
// Largest row norm of C [Nc][d] into *out (zeroed by the caller).
hipError_t launch_cnorm_max(const void* C, int dtype, int Nc, int d, unsigned long long* out,
                            hipStream_t s);
hipError_t launch_scores(const PassArgs& a, hipStream_t s);
hipError_t launch_topk(const PassArgs& a, int mode, hipStream_t s);   // mode: TopkMode
hipError_t launch_gather(const PassArgs& a, int mode, hipStream_t s);
hipError_t launch_topm_merge(const PassArgs& a, hipStream_t s);
hipError_t launch_finalize(const PassArgs& a, hipStream_t s);
// Slot norms of the packed slabs (certified argmax) into out [n_tiles][64].
hipError_t launch_slot_norms(const void* ET, int slab, const float* escale, long n_tiles, int d,
                             float* out, hipStream_t s);
// Size of the static scratch array of ce_top_tokens_static (bytes).
constexpr size_t kStaticScratchBytes = size_t(4) << 20;
// Device address of the static scratch array on the current device (looked
// up with hipGetSymbolAddress on the first call per device).
hipError_t static_scratch(void** ptr);
// Read every 16-byte vector of buf[0, bytes) once (measurement probe).
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);

}  // namespace ce
