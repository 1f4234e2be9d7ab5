// HIP kernels of the centroid-masked sparse LM head, written for CDNA4 (gfx950).
//
// The operation is Gemma4MTPMaskedEmbedder of the vLLM compare view "[Spec
// Decode] Add Gemma4 MTP speculative decoding with centroids masking" (diff of
// gemma4_mtp.py): centroid projection, top-K centroids, gather of the tokens
// the selected centroids own (ordered-embedding layout), sparse dot products,
// then a greedy argmax (get_top_tokens) or a full-vocabulary row filled with
// -inf outside the candidates (forward).
//
// Packed weights.  At prepare time the centroid rows and the ordered
// embedding rows are packed in tiles of 64 rows (a cluster's slots never
// share a tile with another cluster): tile t stores, for every 16-byte vector
// v of a row, the vectors of its 64 rows side by side, [t][v][lane].  Lane l
// of a wave then reads its own row's next 8 bf16 (or 4 fp32) elements while
// the wave reads 1 KiB of contiguous memory, so slabs stream from HBM straight
// into registers, fully coalesced.
//
// One pass handles at most 64 rows and runs these kernels in stream order:
//   scores   centroid projection S[b][c] (canonical dot, see below); for
//            forward it also fills the output rows with -inf
//   topk     one workgroup per row: the K best centroids (a threshold from
//            the waves' maxima, then parallel rank counts among the keys
//            above it); writes the ids and the row's 64-centroid selection
//            words
//   gather   one wave per 64-token tile of the static tile list (two from
//            48 rows, sharing the tile's passes of 4 rows); a tile whose
//            centroid no row selected exits at once, so each selected slab is
//            read exactly once however many rows share it (cross-row dedup).
//            The tile is dotted with every row that selected it, then reduced
//            to a per-row packed argmax (64-bit atomicMax) or stored at the
//            candidates' token columns of the forward rows.  Up to 4 rows
//            with equal clusters, one wave per selected (row, centroid, tile)
//            instead, so no wave is launched for an unselected tile
//   finalize (get_top_tokens) decode the packed argmax into token ids
//
// No kernel waits on another workgroup and none uses a device-scope fence:
// on a multi-XCD part such a fence writes back the L2, so results travel
// between steps only through kernel boundaries and fire-and-forget atomics.
//
// Canonical dot: every product is formed exactly in float64 and summed in
// hidden-dimension order from +0.0 by a chain of v_fmac_f64 (one rounding per
// step), then rounded to fp32 nearest-even with -0 mapped to +0.  Each lane
// owns whole chains (one per output), so no reduction tree reorders a sum and
// the results equal a sequential float64 loop bit for bit.  The hidden rows are
// wave-uniform operands: each lane widens four elements of a 64-dim chunk to
// float64 and a 64-bit DPP row broadcast hands element k to every lane, so
// the hidden rows take no LDS traffic and no barriers.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "ce_internal.h"

// Wavefront reductions and scans of the ROCm device library (DPP based).
extern "C" __device__ unsigned int __ockl_wfred_add_u32(unsigned int);
extern "C" __device__ unsigned int __ockl_wfscan_add_u32(unsigned int, bool inclusive);
extern "C" __device__ unsigned long long __ockl_wfred_max_u64(unsigned long long);
extern "C" __device__ unsigned long long __ockl_wfred_min_u64(unsigned long long);

namespace ce {
namespace {

constexpr int kWave = 64;
constexpr int kChunk = 64;       // hidden dims per register stage
constexpr int kGatherRows = 4;   // hidden rows dotted per pass over a gather tile
constexpr int kGatherSplitShift = 1;   // log2 waves per gather tile for large batches

// 16 bytes as a native vector (HIP's uint4 wraps a union, which keeps arrays
// of it out of registers).
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Weight element types: fp32, bf16 bits, and OCP E4M3 codes (FP8 slabs,
// whose hidden rows stay bf16).
template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int kPerVec = 4; typedef float hidden; };
template <> struct Elem<uint16_t> { static constexpr int kPerVec = 8; typedef uint16_t hidden; };
template <> struct Elem<uint8_t> { static constexpr int kPerVec = 16; typedef uint16_t hidden; };

// 16 bytes of elements -> float64, exactly.
__device__ __forceinline__ void widen(const v4u v, double (&x)[4], float) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = (double)__uint_as_float(v[i]);
}
__device__ __forceinline__ void widen(const v4u v, double (&x)[8], uint16_t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = (double)__uint_as_float(v[i] << 16);
    x[2 * i + 1] = (double)__uint_as_float(v[i] & 0xffff0000u);
  }
}
// E4M3 codes: gfx950's packed conversion decodes OCP E4M3 exactly (all 256
// codes checked against the format's definition).
typedef float v2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void widen(const v4u v, double (&x)[16], uint8_t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[i], false);
    const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[i], true);
    x[4 * i] = (double)lo.x;
    x[4 * i + 1] = (double)lo.y;
    x[4 * i + 2] = (double)hi.x;
    x[4 * i + 3] = (double)hi.y;
  }
}

// float64 sum -> fp32 nearest-even, -0 -> +0.
__device__ __forceinline__ float canon(double s) {
  uint32_t u = __float_as_uint((float)s);
  return __uint_as_float(u == 0x80000000u ? 0u : u);
}

// Keep a loaded value live on every path.  Without it the compiler sinks a
// load whose result is only used under a condition into that branch, and a
// load under a branch is waited for on its own (no overlap with the others).
template <typename V>
__device__ __forceinline__ void pin(V& v) {
  asm volatile("" : "+v"(v));
}

// Order-preserving map of a (non-NaN) fp32 to u32; -0 and +0 map alike.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// fp32 at or above x (x >= 0): the nearest float, raised one step if below.
__device__ __forceinline__ float f32_up(double x) {
  float f = (float)x;
  if ((double)f < x) f = __uint_as_float(__float_as_uint(f) + 1u);
  return f;
}

// Inverse of order_key (a key of -0 does not occur: order_key maps it to +0).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ------------------------------------------------------------------ packing

// Pack rows of W ([rows][d] row-major) into 64-row tiles [t][v][lane].
// With `tiles` (the cluster tile list) tile t covers the slots of one
// cluster's 64-slot tile; without it, tile t covers rows [64t, 64t+64) of
// `nrows_total`.  Lanes past a tile's last row are zero.
__global__ __launch_bounds__(256) void pack_kernel(const v4u* __restrict__ W, int nvec, long n_out,
                                                   const uint32_t* __restrict__ tiles,
                                                   const int32_t* __restrict__ offsets,
                                                   int nrows_total, v4u* __restrict__ out) {
  const long stride = (long)gridDim.x * blockDim.x;
  for (long o = (long)blockIdx.x * blockDim.x + threadIdx.x; o < n_out; o += stride) {
    const int lane = (int)(o % kTileTokens);
    const long tv = o / kTileTokens;
    const int v = (int)(tv % nvec);
    const long t = tv / nvec;
    long start, end;
    if (tiles) {
      const uint32_t w = tiles[t];
      const int c = (int)(w & ((1u << kTileShift) - 1u));
      start = (long)offsets[c] + (long)(w >> kTileShift) * kTileTokens;
      end = offsets[c + 1];
    } else {
      start = t * kTileTokens;
      end = nrows_total;
    }
    const long row = start + lane;
    v4u val = {0u, 0u, 0u, 0u};
    if (row < end) val = W[row * nvec + v];
    out[o] = val;
  }
}

// OCP E4M3 code of a finite float64: nearest, ties to even, magnitudes
// beyond 448 saturate to 448, the sign of zero kept.
__device__ __forceinline__ uint32_t e4m3_rne_sat(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const uint32_t sign = (uint32_t)(u >> 56) & 0x80u;
  const unsigned long long mag = u & 0x7FFFFFFFFFFFFFFFull;
  const double a = __longlong_as_double((long long)mag);
  if (a < 0x1p-6) {
    // subnormal codes k * 2^-9; k = 8 is code 0x08, the smallest normal
    return sign | (uint32_t)rint(a * 512.0);
  }
  int e = (int)(mag >> 52) - 1023;
  const unsigned long long m = (mag & ((1ull << 52) - 1ull)) | (1ull << 52);
  unsigned long long q = m >> 49;                 // leading one and three fraction bits
  const unsigned long long rem = m & ((1ull << 49) - 1ull), half = 1ull << 48;
  if (rem > half || (rem == half && (q & 1ull))) ++q;
  if (q == 16) {
    q = 8;
    ++e;
  }
  if (e > 8 || (e == 8 && q > 14)) return sign | 0x7Eu;
  return sign | ((uint32_t)(e + 7) << 3) | (uint32_t)(q - 8);
}

// Quantise the rows of W (bf16, [rows][d] row-major) to E4M3 with one float32
// scale per row, s = fl32(max |w| / 448) (1 for a zero row), codes
// E4M3(fl64(w / s)), and pack them like pack_kernel: tile t of the cluster
// tile list, or rows [64t, 64t+64) without one, [t][d/16][lane] vectors of
// 16 codes, scale[t][lane].  One thread per tile row; lanes past a tile's
// last row get zero codes and scale.
__global__ __launch_bounds__(256) void pack_fp8_kernel(const uint16_t* __restrict__ W, int d,
                                                       long n_rows_out,
                                                       const uint32_t* __restrict__ tiles,
                                                       const int32_t* __restrict__ offsets,
                                                       long nrows_total,
                                                       v4u* __restrict__ out,
                                                       float* __restrict__ scale) {
  const int nvec = d / 16;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long o = (long)blockIdx.x * blockDim.x + threadIdx.x; o < n_rows_out; o += stride) {
    const int lane = (int)(o % kTileTokens);
    const long t = o / kTileTokens;
    long row, end;
    if (tiles) {
      const uint32_t w = tiles[t];
      const int c = (int)(w & ((1u << kTileShift) - 1u));
      row = (long)offsets[c] + (long)(w >> kTileShift) * kTileTokens + lane;
      end = offsets[c + 1];
    } else {
      row = t * kTileTokens + lane;
      end = nrows_total;
    }
    v4u* dst = out + t * (long)nvec * kTileTokens + lane;
    if (row >= end) {
      for (int v = 0; v < nvec; ++v) dst[(long)v * kTileTokens] = v4u{0u, 0u, 0u, 0u};
      scale[o] = 0.0f;
      continue;
    }
    const uint16_t* x = W + row * d;
    float amax = 0.0f;
    for (int k = 0; k < d; ++k) amax = fmaxf(amax, fabsf(__uint_as_float((uint32_t)x[k] << 16)));
    // fl64 then fl32 of amax/448 equals the correctly rounded float32
    // quotient: for a bf16 amax it is exact or far from a float32 midpoint
    const float s = amax > 0.0f ? (float)((double)amax / 448.0) : 1.0f;
    const double sd = (double)s;
    for (int v = 0; v < nvec; ++v) {
      v4u q;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t word = 0u;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const double xv = (double)__uint_as_float((uint32_t)x[16 * v + 4 * i + b] << 16);
          word |= e4m3_rne_sat(xv / sd) << (8 * b);
        }
        q[i] = word;
      }
      dst[(long)v * kTileTokens] = q;
    }
    scale[o] = s;
  }
}

// ------------------------------------------------------------------ dot tile

// acc = fma(h_k, x_k, acc) for the elements k of one weight vector, in
// order, with h_k taken from lane k/4 of this lane's 16-lane row by a 64-bit
// DPP row broadcast fused into v_fmac_f64 (src0), so the hidden value costs
// neither LDS traffic nor an extra instruction.  hq holds this lane's four
// elements.  A DPP read needs two wait states after a VALU write of its
// source; the compiler cannot see inside the asm, so each block starts with
// them.
template <int J>
__device__ __forceinline__ void fmac_vec(double& acc, const double (&hq)[4], const double (&x)[8]) {
  // bf16: elements 8p..8p+7 sit in lanes J = 2p (first four) and J+1
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f64_dpp %0, %1, %5 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %2, %6 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %3, %7 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %4, %8 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %1, %9 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %2, %10 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %3, %11 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %4, %12 row_newbcast:%14 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(hq[0]), "v"(hq[1]), "v"(hq[2]), "v"(hq[3]), "v"(x[0]), "v"(x[1]), "v"(x[2]),
        "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "n"(J), "n"(J + 1));
}
template <int J>
__device__ __forceinline__ void fmac_vec(double& acc, const double (&hq)[4], const double (&x)[4]) {
  // fp32: elements 4p..4p+3 sit in lane J = p
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f64_dpp %0, %1, %5 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %2, %6 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %3, %7 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %4, %8 row_newbcast:%9 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(hq[0]), "v"(hq[1]), "v"(hq[2]), "v"(hq[3]), "v"(x[0]), "v"(x[1]), "v"(x[2]),
        "v"(x[3]), "n"(J));
}
template <int J>
__device__ __forceinline__ void fmac_vec(double& acc, const double (&hq)[4], const double (&x)[16]) {
  // E4M3: elements 16p..16p+15 sit in lanes J = 4p .. 4p+3, four each
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f64_dpp %0, %1, %5 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %2, %6 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %3, %7 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %4, %8 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %1, %9 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %2, %10 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %3, %11 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %4, %12 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %1, %13 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %2, %14 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %3, %15 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %4, %16 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %1, %17 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %2, %18 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %3, %19 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %4, %20 row_newbcast:%24 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(hq[0]), "v"(hq[1]), "v"(hq[2]), "v"(hq[3]), "v"(x[0]), "v"(x[1]), "v"(x[2]),
        "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]),
        "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]), "n"(J),
        "n"(J + 1), "n"(J + 2), "n"(J + 3));
}
// f(std::integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Four consecutive hidden-row elements as loaded by one lane.
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
template <typename T> struct HQuad;
template <> struct HQuad<uint16_t> { typedef v2u raw; };   // 4 bf16
template <> struct HQuad<float> { typedef v4u raw; };      // 4 fp32

__device__ __forceinline__ void widen4(const v2u r, double (&x)[4]) {
  x[0] = (double)__uint_as_float(r[0] << 16);
  x[1] = (double)__uint_as_float(r[0] & 0xffff0000u);
  x[2] = (double)__uint_as_float(r[1] << 16);
  x[3] = (double)__uint_as_float(r[1] & 0xffff0000u);
}
__device__ __forceinline__ void widen4(const v4u r, double (&x)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = (double)__uint_as_float(r[i]);
}

// Dot one packed 64-row tile `wt` ([d/kPerVec][64] vectors, zero-padded)
// with the hidden rows h[rows[r]] for r < nrows ([*][d] of T).  Lane t ends
// with acc[r] = the float64 chain of (tile row t, hidden row rows[r]).
//
// Per chunk of 64 dims each lane loads its tile row's vectors (one 1 KiB
// coalesced wave load per vector) one chunk ahead of use, and four
// consecutive elements of each hidden row: lane l of every 16-lane row holds
// elements 4l..4l+3 of the chunk, widened to float64, and element k reaches
// every lane by a 64-bit DPP broadcast from lane k/4 of its row.
struct NoOp {
  __device__ void operator()() const {}
};

// Buffer range of a tile for predicated loads: a lane whose byte offset is
// at or past it reads zeros and fetches nothing.  Tiles are far smaller.
constexpr uint32_t kBufRange = 0x40000000u;
constexpr uint32_t kBufWord3 = 0x00020000u;   // raw buffer, 32-bit data format

// With SPLIT (a compile-time chunk count only), the first stages' tile loads
// are issued, then mid() runs, then the first stages' hidden loads: mid may
// produce the hidden rows (in LDS) while the tile loads are in flight.
// With PRED the tile is read by buffer loads at lane_off (the lane's byte
// offset 16 * lane, or kBufRange beyond it for a lane that needs no row), so
// the slots no row needs cost no memory traffic.
template <typename T, int RB, int NCH, int STAGES = 2, bool SPLIT = false, typename Mid = NoOp,
          bool STREAM = false, bool PRED = false>
__device__ __forceinline__ void dot_tile(const v4u* __restrict__ wt, int d,
                                         const typename Elem<T>::hidden* __restrict__ h,
                                         const int (&rows)[RB], int nrows, double (&acc)[RB],
                                         Mid&& mid = Mid(), uint32_t lane_off = 0u) {
  using TH = typename Elem<T>::hidden;
  constexpr int PV = Elem<T>::kPerVec;
  constexpr int VPC = kChunk / PV;              // weight vectors per chunk
  using HR = typename HQuad<TH>::raw;
  const int lane = threadIdx.x;
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = 0.0;
  const TH* hp[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) hp[r] = h + (long)rows[r] * d + 4 * (lane & 15);

  // Every load is unconditional (packed tiles are zero-padded to 64 rows and
  // hidden-row slots are clamped to valid rows): a load under a branch makes
  // the compiler wait for all outstanding loads at the join, which would
  // serialise the two stages in flight.
  struct Stage {
    v4u e[VPC];
    HR h[RB];
  };
  __amdgpu_buffer_rsrc_t rsrc;
  if constexpr (PRED)
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<v4u*>(wt), (short)0, (int)kBufRange,
                                             (int)kBufWord3);
  auto load_w = [&](Stage& st, int ch) {
#pragma unroll
    for (int p = 0; p < VPC; ++p) {
      // STREAM: tiles read once per call (the gather's slabs) skip the caches
      if constexpr (PRED)
        st.e[p] = __builtin_amdgcn_raw_buffer_load_b128(
            rsrc, lane_off + (uint32_t)((ch * VPC + p) * kWave * 16), 0, STREAM ? 2 : 0);
      else if constexpr (STREAM) st.e[p] = __builtin_nontemporal_load(&wt[(ch * VPC + p) * kWave + lane]);
      else st.e[p] = wt[(ch * VPC + p) * kWave + lane];
    }
  };
  auto load_h = [&](Stage& st, int ch) {
#pragma unroll
    for (int r = 0; r < RB; ++r) st.h[r] = *reinterpret_cast<const HR*>(hp[r] + ch * kChunk);
  };
  auto load = [&](Stage& st, int ch) {
    load_w(st, ch);
    load_h(st, ch);
  };
  auto consume = [&](const Stage& st) {
    double hd[RB][4];
#pragma unroll
    for (int r = 0; r < RB; ++r) widen4(st.h[r], hd[r]);
    static_for<0, VPC>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      double x[PV];
      widen(st.e[p], x, T());
#pragma unroll
      for (int r = 0; r < RB; ++r)
        if (r < nrows) fmac_vec<p * PV / 4>(acc[r], hd[r], x);
      // widen each vector right before its use (hoisting them all would
      // hold a whole chunk of float64 weights in registers)
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // A ring of register stages: while one chunk is consumed the next
  // STAGES-1 are in flight; a stage is reloaded only after it has been
  // consumed.  With the chunk count NCH known at compile time the pipeline
  // is straight-line code; otherwise two stages, where the steady-state loop
  // (even chunk counts) reloads unconditionally and the last two chunks are
  // peeled, so no load sits under a branch.
  if constexpr (NCH > 0) {
    constexpr int S = STAGES < NCH ? STAGES : NCH;
    Stage st[S];
    // scheduling barriers keep each stage's loads together and in order, so
    // that waiting for one stage never waits for the next
    if constexpr (SPLIT) {
      static_for<0, S>([&](auto i) {
        load_w(st[decltype(i)::value], decltype(i)::value);
        __builtin_amdgcn_sched_barrier(0);
      });
      mid();
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, S>([&](auto i) { load_h(st[decltype(i)::value], decltype(i)::value); });
      __builtin_amdgcn_sched_barrier(0);
    } else {
      static_for<0, S>([&](auto i) {
        load(st[decltype(i)::value], decltype(i)::value);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    static_for<0, NCH>([&](auto c) {
      constexpr int ch = decltype(c)::value;
      consume(st[ch % S]);
      if constexpr (ch + S < NCH) load(st[ch % S], ch + S);
      __builtin_amdgcn_sched_barrier(0);
    });
    return;
  }
  Stage s0, s1;
  const int nch = d / kChunk;
  if (nch == 1) {
    load(s0, 0);
    consume(s0);
  } else if ((nch & 1) == 0) {
    load(s0, 0);
    load(s1, 1);
    for (int ch = 0; ch < nch - 2; ch += 2) {
      consume(s0);
      load(s0, ch + 2);
      consume(s1);
      load(s1, ch + 3);
    }
    consume(s0);
    consume(s1);
  } else {
    load(s0, 0);
    load(s1, 1);
    for (int ch = 0; ch < nch; ch += 2) {
      consume(s0);
      if (ch + 2 < nch) load(s0, ch + 2);
      if (ch + 1 < nch) {
        consume(s1);
        if (ch + 3 < nch) load(s1, ch + 3);
      }
    }
  }
}

// ------------------------------------------------------------------ final norm

// float32 -> bf16 bits, nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Four normalised elements, stored as the head's element type.
__device__ __forceinline__ v2u pack_norm(const double (&y)[4], uint16_t) {
  v2u o;
  o[0] = bf16_rne((float)y[0]) | (bf16_rne((float)y[1]) << 16);
  o[1] = bf16_rne((float)y[2]) | (bf16_rne((float)y[3]) << 16);
  return o;
}
__device__ __forceinline__ v4u pack_norm(const double (&y)[4], float) {
  v4u o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __float_as_uint((float)y[i]);
  return o;
}

struct NormArgs {
  const void* w;       // [d] norm weight, head dtype
  double eps;          // widened from float32
  void* out;           // [B][d] normalised rows, head dtype
};

// ss = fl64(ss + q_k) for the four squares q[0..3] held by lane J of this
// lane's 16-lane row, in order: a 64-bit DPP row broadcast fused into
// v_fmac_f64 with src1 = 1.0, so each step is the sum's single rounding
// (q * 1 is exact).  The two wait states a DPP read needs after the VALU
// write of its source open the block.
template <int J>
__device__ __forceinline__ void sq_add4(double& ss, const double (&q)[4], const double& one) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f64_dpp %0, %1, %5 row_newbcast:%6 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %2, %5 row_newbcast:%6 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %3, %5 row_newbcast:%6 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %4, %5 row_newbcast:%6 row_mask:0xf bank_mask:0xf"
      : "+v"(ss)
      : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(one), "n"(J));
}

// Add the 64 squares of one chunk to ss in element order.  Every 16-lane
// row of the wave holds the same chunk (lane l: elements 4(l%16) .. +3), so
// every lane runs the same chain and ends with the same sum.
template <typename HR>
__device__ __forceinline__ void sq_chunk(double& ss, const HR xr) {
  double x[4], q[4];
  widen4(xr, x);
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = x[i] * x[i];   // exact in float64
  const double one = 1.0;
  static_for<0, 16>([&](auto j) { sq_add4<decltype(j)::value>(ss, q, one); });
}

// y = (x r) w for four elements, stored to LDS and (given out) to out.
template <typename T, typename HR>
__device__ __forceinline__ void norm_store(const HR xr, const HR wr, double rr, T* lds,
                                           T* __restrict__ out) {
  double xv[4], wv[4], y[4];
  widen4(xr, xv);
  widen4(wr, wv);
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = (xv[i] * rr) * wv[i];
  const HR o = pack_norm(y, T());
  *reinterpret_cast<HR*>(lds) = o;
  if (out) *reinterpret_cast<HR*>(out) = o;
}

// The final RMSNorm of the rows rows[0..RB) of x ([*][d]), written to
// lds ([RB][d], slot r for rows[r]) and, given `out`, to out[rows[r]] for
// r < nrows.  Canonical rounding: the sum of squares is the sequential
// float64 chain ss = fl64(ss + x_k^2) over k in order from +0.0 (squares
// exact); v = ss / d + eps, r = 1 / sqrt(v), y = (x r) w, each one correctly
// rounded float64 operation; y is rounded to float32 and then to the head's
// element type (nearest, ties to even).
//
// The chain runs in every lane (see sq_chunk); lane l then writes chunks
// c = l/16 (mod 4), elements 4(l%16) .. +3.
template <typename T, int RB>
__device__ __forceinline__ void normalize_rows(const T* __restrict__ x, const int (&rows)[RB],
                                               int nrows, int d, const NormArgs& nm,
                                               T* lds, T* __restrict__ out) {
  using HR = typename HQuad<T>::raw;
  const int lane = threadIdx.x;
  const int g = lane >> 4;
  const int e4 = 4 * (lane & 15);
  const int nch = d / kChunk;
  const T* w = static_cast<const T*>(nm.w);
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const T* xr = x + (long)rows[r] * d;
    double ss = 0.0;
    for (int c = 0; c < nch; ++c) sq_chunk(ss, *reinterpret_cast<const HR*>(xr + c * kChunk + e4));
    const double rr = 1.0 / sqrt(ss / (double)d + nm.eps);
    for (int c = g; c < nch; c += 4) {
      const int k = c * kChunk + e4;
      norm_store<T>(*reinterpret_cast<const HR*>(xr + k), *reinterpret_cast<const HR*>(w + k), rr,
                    lds + r * d + k, out && r < nrows ? out + (long)rows[r] * d + k : nullptr);
    }
  }
}

// The same norm with its loads split from its arithmetic, for a chunk
// count NCH known at compile time: norm_load issues the rows' loads (every
// chunk, as the chain reads them) and the weight's (the chunks this lane
// writes), norm_finish does the rest, so that other loads go out in between.
template <typename T, int RB, int NCH>
struct NormRegs {
  static constexpr int NW = (NCH + 3) / 4;
  typename HQuad<T>::raw x[RB][NCH];   // every chunk, as the chain reads them
  typename HQuad<T>::raw xs[RB][NW];   // the chunks 4q + l/16 this lane writes
  typename HQuad<T>::raw w[NW];
};

template <typename T, int RB, int NCH>
__device__ __forceinline__ void norm_load(NormRegs<T, RB, NCH>& nr, const T* __restrict__ x,
                                          const int (&rows)[RB], int d, const NormArgs& nm) {
  using HR = typename HQuad<T>::raw;
  const int lane = threadIdx.x;
  const int g = lane >> 4;
  const int e4 = 4 * (lane & 15);
  const T* w = static_cast<const T*>(nm.w);
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int r = 0; r < RB; ++r)
      nr.x[r][c] = *reinterpret_cast<const HR*>(x + (long)rows[r] * d + c * kChunk + e4);
  // the lane's own chunks are loaded once more (cache hits) rather than
  // picked out of nr.x by a lane-dependent index, which would go to scratch
#pragma unroll
  for (int q = 0; q < NormRegs<T, RB, NCH>::NW; ++q) {   // clamped: unconditional loads
    const int k = min(4 * q + g, NCH - 1) * kChunk + e4;
#pragma unroll
    for (int r = 0; r < RB; ++r) nr.xs[r][q] = *reinterpret_cast<const HR*>(x + (long)rows[r] * d + k);
    nr.w[q] = *reinterpret_cast<const HR*>(w + k);
  }
}

template <typename T, int RB, int NCH>
__device__ __forceinline__ void norm_finish(const NormRegs<T, RB, NCH>& nr, const int (&rows)[RB],
                                            int nrows, int d, const NormArgs& nm, T* lds,
                                            T* __restrict__ out) {
  using HR = typename HQuad<T>::raw;
  const int lane = threadIdx.x;
  const int g = lane >> 4;
  const int e4 = 4 * (lane & 15);
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    double ss = 0.0;
    static_for<0, NCH>([&](auto c) { sq_chunk(ss, nr.x[r][decltype(c)::value]); });
    const double rr = 1.0 / sqrt(ss / (double)d + nm.eps);
#pragma unroll
    for (int q = 0; q < NormRegs<T, RB, NCH>::NW; ++q) {
      const int c = 4 * q + g;
      if (c < NCH) {
        const int k = c * kChunk + e4;
        norm_store<T>(nr.xs[r][q], nr.w[q], rr, lds + r * d + k,
                      out && r < nrows ? out + (long)rows[r] * d + k : nullptr);
      }
    }
  }
}

// ------------------------------------------------------------------ scores

// Forward: -inf over out[0..n) (16-byte aligned), the share of fill group f
// of nfill, groups of NT threads: runs of NT float4 (16 B a thread),
// strided over the groups.  Plain streaming stores.
template <int NT>
__device__ __forceinline__ void fill_share(float* __restrict__ out, long n, long f, long nfill) {
  const int t = threadIdx.x;
  const float ninf = -__builtin_inff();
  const long n4 = n / 4;
  for (long i = f * NT + t; i < n4; i += nfill * NT)
    reinterpret_cast<float4*>(out)[i] = make_float4(ninf, ninf, ninf, ninf);
  if (f == 0)
    for (long i = 4 * n4 + t; i < n; i += NT) out[i] = ninf;
}

// The forward's -inf fill is shared between the projection kernel and the
// top-K kernel, whose one workgroup per row leaves most CUs idle: the
// projection's waves fill out[0, fill_split) and extra top-K workgroups the
// rest.  Both kernels are otherwise latency- or VALU-bound, so each hides
// its share of the stores.
constexpr int kFillProjPct = 50;
__host__ __device__ inline long fill_split(long n) { return (n * kFillProjPct / 100) & ~3l; }

// One wave per (64-centroid tile, RB rows): S[b][c] for the tile's
// centroids.  With `fill` (forward) the grid has more rows of workgroups
// than row groups: those waves fill the output rows with -inf while the
// others compute (a wave that did both would wait for its stores at every
// load: stores and loads share one counter).
//
// With NORM, h holds the rows before the final RMSNorm: the wave normalises
// its rows into LDS (dynamic, [RB][d]) and dots the tile with those; the
// waves of the first centroid tile also write them to nm.out.
template <typename T, int RB, int NCH, bool NORM>
__global__ __launch_bounds__(64) void scores_kernel(const v4u* __restrict__ CT, int Nc, int d,
                                                    const T* __restrict__ h, int B,
                                                    float* __restrict__ S, int ldS,
                                                    float* __restrict__ fill, int V,
                                                    NormArgs nm) {
  extern __shared__ __attribute__((aligned(16))) unsigned char norm_lds[];
  const int lane = threadIdx.x;
  const int c0 = blockIdx.x * kTileTokens;
  const int r0 = blockIdx.y * RB;
  const int nvalid = min(kTileTokens, Nc - c0);
  const int ngroups = (B + RB - 1) / RB;
  if ((int)blockIdx.y >= ngroups) {
    fill_share<kWave>(fill, fill_split((long)B * V), (long)(blockIdx.y - ngroups) * gridDim.x + blockIdx.x,
                      (long)(gridDim.y - ngroups) * gridDim.x);
    return;
  }
  const int nrows = min(RB, B - r0);
  int rows[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) rows[r] = r0 + (r < nrows ? r : nrows - 1);
  double acc[RB];
  const long tile_vecs = (long)(d / Elem<T>::kPerVec) * kWave;
  if constexpr (NORM) {
    T* hn = reinterpret_cast<T*>(norm_lds);
    T* out = blockIdx.x == 0 ? static_cast<T*>(nm.out) : nullptr;
    int lrows[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) lrows[r] = r < nrows ? r : 0;
    if constexpr (NCH > 0) {
      // row and weight loads first, then the tile's first stages; the norm
      // is computed while those are in flight
      NormRegs<T, RB, NCH> nr;
      norm_load<T, RB, NCH>(nr, h, rows, d, nm);
      __builtin_amdgcn_sched_barrier(0);
      dot_tile<T, RB, NCH, 2, true>(CT + blockIdx.x * tile_vecs, d, hn, lrows, nrows, acc, [&] {
        norm_finish<T, RB, NCH>(nr, rows, nrows, d, nm, hn, out);
        __syncthreads();
      });
    } else {
      normalize_rows<T, RB>(h, rows, nrows, d, nm, hn, out);
      __syncthreads();
      dot_tile<T, RB, NCH>(CT + blockIdx.x * tile_vecs, d, hn, lrows, nrows, acc);
    }
  } else {
    // two rows a wave (the forward from 48 rows, beside its fill waves):
    // three stages of the centroid tile in flight (forward B=64: 46.2 ->
    // 45.1 µs per call); one row a wave keeps two (three cost the B=64
    // argmax 0.2 µs)
    dot_tile<T, RB, NCH, RB >= 2 ? 3 : 2>(CT + blockIdx.x * tile_vecs, d, h, rows, nrows, acc);
  }
  if (lane < nvalid) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
      if (r < nrows) S[(long)(r0 + r) * ldS + c0 + lane] = canon(acc[r]);
  }
}

// ------------------------------------------------------------------ approximate scores (MFMA)

// bf16 operands of v_mfma_f32_16x16x32_bf16 and its fp32 accumulator.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Approximate centroid scores of a bf16 head, for the certified top-K:
// S~[b][c] = sum_k h[b][k] C[c][k] accumulated by the matrix cores in fp32,
// whatever their internal order.  One wave per (16 MB centroids, 16 rows):
// per k-step of 32 the A operands are MB blocks of 16 centroid rows (lane l:
// row l%16, elements 8(l/16) .. +7, one 16-byte vector of the packed tile)
// and the B operand 16 hidden rows the same way; lane l ends with
// D[4(l/16) + i][l%16], the scores of centroids 4(l/16) + i of each block
// for hidden row l%16.  With `fill` (forward) the extra grid rows stream
// -inf over the output rows, as in scores_kernel.
template <int MB, int NKS>
__global__ __launch_bounds__(64) void proj_mfma_kernel(const v4u* __restrict__ CT, int Nc, int d,
                                                       const uint16_t* __restrict__ h, int B,
                                                       float* __restrict__ S, int ldS,
                                                       float* __restrict__ fill, int V) {
  const int lane = threadIdx.x;
  const int ngroups = (B + 15) / 16;
  if ((int)blockIdx.y >= ngroups) {
    fill_share<kWave>(fill, fill_split((long)B * V), (long)(blockIdx.y - ngroups) * gridDim.x + blockIdx.x,
                      (long)(gridDim.y - ngroups) * gridDim.x);
    return;
  }
  const int r = lane & 15, kq = lane >> 4;
  const int c0 = blockIdx.x * 16 * MB;
  const int row0 = blockIdx.y * 16;
  const int nks = NKS > 0 ? NKS : d / 32;
  const int nvec = d / 8;
  // unconditional loads: hidden rows past B repeat row B-1, and centroid
  // rows past Nc read the packed tiles' zero padding
  const v4u* hp = reinterpret_cast<const v4u*>(h + (long)min(row0 + r, B - 1) * d) + kq;
  const v4u* cp[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int c = c0 + 16 * m + r;
    cp[m] = CT + ((long)(c / kTileTokens) * nvec + kq) * kWave + (c % kTileTokens);
  }
  v4f acc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
  // groups of G k-steps in a ring of two register stages: the next group's
  // loads are in flight while a group's MFMAs run (clamped, so
  // unconditional; the MFMAs of steps past the end are skipped)
  constexpr int G = 4;
  struct Stage {
    v4u b[G], a[G][MB];
  };
  auto load = [&](Stage& st, int s0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int s = min(s0 + j, nks - 1);
      st.b[j] = hp[4 * s];
#pragma unroll
      for (int m = 0; m < MB; ++m) st.a[j][m] = cp[m][(long)4 * s * kWave];
    }
  };
  auto run = [&](const Stage& st, int s0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (s0 + j < nks) {
#pragma unroll
        for (int m = 0; m < MB; ++m)
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, st.a[j][m]),
                                                           __builtin_bit_cast(v8bf, st.b[j]),
                                                           acc[m], 0, 0, 0);
      }
    }
  };
  Stage st0, st1;
  load(st0, 0);
  if (nks > G) load(st1, G);
#pragma unroll
  for (int s0 = 0; s0 < nks; s0 += 2 * G) {
    run(st0, s0);
    if (s0 + 2 * G < nks) load(st0, s0 + 2 * G);
    if (s0 + G < nks) {
      run(st1, s0 + G);
      if (s0 + 3 * G < nks) load(st1, s0 + 3 * G);
    }
  }
  const int row = row0 + r;
  if (row < B) {
    float* out = S + (long)row * ldS;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int c = c0 + 16 * m + 4 * kq;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (c + i < Nc) out[c + i] = acc[m][i];
    }
  }
}

// Largest row norm of the centroids, rounded up, max-ed into *out as the
// bits of a positive double (ordered like unsigned integers); *out starts
// at 0.  The row's sum of squares is a float64 chain (relative error below
// d 2^-53), and the square root is scaled by 1 + 2^-40, which covers it.
template <typename T>
__global__ __launch_bounds__(256) void cnorm_max_kernel(const T* __restrict__ C, int Nc, int d,
                                                        unsigned long long* __restrict__ out) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  double ss = 0.0;
  if (c < Nc) {
    for (int k = 0; k < d; ++k) {
      double x;
      if constexpr (std::is_same<T, uint16_t>::value) x = (double)__uint_as_float((uint32_t)C[(long)c * d + k] << 16);
      else x = (double)C[(long)c * d + k];
      ss = fma(x, x, ss);
    }
  }
  const double n = sqrt(ss) * (1.0 + 0x1p-40);
  const unsigned long long bits = __ockl_wfred_max_u64((unsigned long long)__double_as_longlong(n));
  if ((threadIdx.x & (kWave - 1)) == 0) atomicMax(out, bits);
}

// ------------------------------------------------------------------ top-K

// Threads of a top-K (and top-m merge) workgroup: 512 measured faster than
// 256 (B=1 15.5 → 15.1 µs per call, B=64 36.9 → 36.7) and than 1024 (16.6,
// 38.4): more waves shorten the per-thread passes until barriers dominate.
constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / kWave;
static_assert(kMaxNc <= 16 * kTopkThreads, "a top-K thread holds at most 16 keys");
constexpr int kCandCap = 1024;   // candidate keys kept for the exact select

// Lanes of the wave below this one whose bit is set in `m`.
__device__ __forceinline__ uint32_t lanes_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t popc64(unsigned long long m) { return (uint32_t)__popcll(m); }

// Exclusive prefix sum over the threads of the block; *total gets the sum.
template <int NW = kTopkWaves>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const uint32_t x = __ockl_wfscan_add_u32(v, false);   // exclusive, within the wave
  if (lane == kWave - 1) sh[w] = x + v;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t s = sh[i];
    base += (i < w) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x;
}

// K-th largest, counting repeats, of the values r[0..NV) of every lane of
// the wave (0 marks an absent value; K must not exceed the present ones), by
// radix select from the top bit: at each bit the values that agree with the
// answer on the bits above and have a 1 at this bit are counted; if they are
// at least kk the answer has a 1 there, else they all rank above it and kk
// drops by their number.  *quota gets kk at the end: how many copies of the
// answer the K largest hold.  All 32 steps are unrolled and branch-free (one
// wave alone runs this, so every taken branch would be paid in full).
template <int NV>
__device__ __forceinline__ uint32_t radix_kth(const uint32_t (&r)[NV], uint32_t K, uint32_t* quota) {
  uint32_t prefix = 0, kk = K;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t want = (prefix >> bit) | 1u;
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) c += popc64(__ballot((r[j] >> bit) == want));
    const bool one = c >= kk;
    prefix |= one ? (1u << bit) : 0u;
    kk -= one ? 0u : c;
  }
  *quota = kk;
  return prefix;
}

// The K-th largest T of cand[0..n) (LDS, nonzero, K <= n), the number of
// copies of T the K largest hold (*quota) and the number of copies in all
// (*copies); one wave.
template <int NV>
__device__ __forceinline__ uint32_t cand_kth(const uint32_t* cand, int n, uint32_t K,
                                             uint32_t* quota, uint32_t* copies) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t r[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int idx = j * kWave + lane;
    r[j] = idx < n ? cand[idx] : 0u;
  }
  const uint32_t T = radix_kth<NV>(r, K, quota);
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) c += popc64(__ballot(r[j] == T));
  *copies = c;
  return T;
}

enum SelectMode { kSelIds = 1, kSelMark = 2 };

struct TopkArgs {
  const float* S;
  int ldS, Nc, K;
  int32_t* out;                    // [rows][ldK] ascending ids
  int ldK;
  unsigned long long* cl_sel;      // [ceil(Nc/64)][64]: bit i of word (w, b) = row b selected 64w+i
  unsigned long long* best;        // [64] top-m counters, cleared per row (or null)
  unsigned long long* amax;        // argmax slots (kArgSlots per row), cleared per row (or null)
  int16_t* rank;                   // [rows][ldR] output position of each selected id (RANK)
  int ldR;
  // approximate scores (APPROX): S holds the matrix cores' fp32 sums, each
  // within E of its canonical key (E from the row's norm and the largest
  // centroid norm); canonical keys are recomputed from h and the packed
  // centroids where the bound leaves the selection open
  const uint16_t* h;               // [rows][d] bf16 hidden rows
  const v4u* CT;                   // packed centroids [ceil(Nc/64)][d/8][64]
  int d;
  const unsigned long long* cmax;  // largest centroid row norm (bits of a double)
  unsigned long long* stats;       // [0] rows whose band was recomputed, [1] rows recomputed whole
  float* hnorm;                    // certified argmax: each row's |h|, rounded up (or null)
  // forward: workgroups from `rows` on fill out[fill_split(n), n) with -inf
  int rows;
  float* fill;
  long fill_n;
};

// Number of the values vals[0..n) (LDS, read as broadcasts; n a multiple
// of kCountBlock, zero-padded) that are greater than x.  Each block of reads
// is issued before the first compare.
constexpr int kCountBlock = 32;
__device__ __forceinline__ uint32_t count_above(const uint32_t* vals, int n, uint32_t x) {
  uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 0;
  for (int j = 0; j < n; j += kCountBlock) {
    v4u q[kCountBlock / 4];
#pragma unroll
    for (int u = 0; u < kCountBlock / 4; ++u) q[u] = *reinterpret_cast<const v4u*>(vals + j + 4 * u);
#pragma unroll
    for (int u = 0; u < kCountBlock / 4; ++u) {
      c0 += q[u].x > x ? 1u : 0u;
      c1 += q[u].y > x ? 1u : 0u;
      c2 += q[u].z > x ? 1u : 0u;
      c3 += q[u].w > x ? 1u : 0u;
    }
  }
  return (c0 + c1) + (c2 + c3);
}

// Exponent of the last significant bit of a bf16 value (nonzero): its
// integer significand is a multiple of 2^this.
__device__ __forceinline__ int bf16_lsb_exp(uint32_t bits) {
  const int e = (int)((bits >> 7) & 0xFFu);
  return e == 0 ? -133 : e - 134;
}

// The canonical key of centroid c (order_key of the canonical dot with the
// bf16 row in LDS), by one whole wave; every lane returns it.  Lane l takes
// the row's 16-byte vectors l and l + 64 of each pass of 128 (one load round
// trip per pass; a single pass up to d = 1024).  Every product is exact in
// float64 and a multiple of 2^q, q the smallest exponent of a product's last
// significant bit; when the sum of their magnitudes is below 2^(q+53),
// every partial sum in any order is a multiple of 2^q below 2^(q+53), so
// exact: the sequential chain then equals the exact sum, which the wave adds
// in parallel.  Otherwise the chain runs in hidden-dimension order, each
// vector broadcast from its lane.
__device__ uint32_t wave_row_key(const v4u* __restrict__ row, const uint16_t* hl, int d) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nvec = d / 8;
  auto prod = [&](const v4u& hv, const v4u& cv, int e) {
    const uint32_t hb = (hv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    const uint32_t cb = (cv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    return (double)__uint_as_float(hb << 16) * (double)__uint_as_float(cb << 16);
  };
  double part = 0.0, mag = 0.0;
  int q = 0x7FFFFFFF;
#pragma unroll 1
  for (int v0 = 0; v0 < nvec; v0 += 2 * kWave) {
    v4u cv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) cv[j] = row[(long)min(v0 + lane + kWave * j, nvec - 1) * kWave];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int v = v0 + lane + kWave * j;
      if (v < nvec) {
        const v4u hv = *reinterpret_cast<const v4u*>(hl + 8 * v);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double p = prod(hv, cv[j], e);
          if (p != 0.0) {
            const uint32_t hb = (hv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            const uint32_t cb = (cv[j][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            part += p;
            mag += fabs(p);
            q = min(q, bf16_lsb_exp(hb) + bf16_lsb_exp(cb));
          }
        }
      }
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    part += __shfl_xor(part, o);
    mag += __shfl_xor(mag, o);
    q = min(q, __shfl_xor(q, o));
  }
  // every lane holds the same sums now (a butterfly), so the test is uniform
  if (q == 0x7FFFFFFF || mag * (1.0 + 0x1p-30) < ldexp(1.0, q + 53)) return order_key(canon(part));
  double acc = 0.0;
#pragma unroll 4
  for (int v = 0; v < nvec; ++v) {
    const v4u cv = row[(long)v * kWave];   // the same address in every lane
    const v4u hv = *reinterpret_cast<const v4u*>(hl + 8 * v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fma((double)__uint_as_float(((hv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16),
                                          (double)__uint_as_float(((cv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16), acc);
  }
  return order_key(canon(acc));
}
__device__ __forceinline__ uint32_t wave_canonical_key(int c, const uint16_t* hl, const v4u* __restrict__ CT,
                                                       int d) {
  return wave_row_key(CT + (long)(c / kTileTokens) * (d / 8) * kWave + (c % kTileTokens), hl, d);
}

// Exponent of the last significant bit of a nonzero decoded E4M3 value
// (at most four significant bits; subnormal codes are multiples of 2^-9).
__device__ __forceinline__ int e4m3_lsb_exp(float f) { return max(ilogbf(f) - 3, -9); }

// The same for a slot of an FP8 slab (vector v = 16 codes at row[64 v]) and
// its row scale: the key of canon(chain * scale), the chain of the bf16
// row's elements times the decoded codes (exact products), by the same
// exact-sum test.
__device__ uint32_t wave_row_key_fp8(const v4u* __restrict__ row, const uint16_t* hl, int d, float sc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nvec = d / 16;
  double part = 0.0, mag = 0.0;
  int q = 0x7FFFFFFF;
#pragma unroll 1
  for (int v0 = 0; v0 < nvec; v0 += kWave) {
    const int v = v0 + lane;
    if (v < nvec) {
      const v4u cv = row[(long)v * kWave];
      double x[16];
      widen(cv, x, uint8_t());
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t hb = hl[16 * v + e];
        const double p = (double)__uint_as_float(hb << 16) * x[e];
        if (p != 0.0) {
          part += p;
          mag += fabs(p);
          q = min(q, bf16_lsb_exp(hb) + e4m3_lsb_exp((float)x[e]));
        }
      }
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    part += __shfl_xor(part, o);
    mag += __shfl_xor(mag, o);
    q = min(q, __shfl_xor(q, o));
  }
  if (q == 0x7FFFFFFF || mag * (1.0 + 0x1p-30) < ldexp(1.0, q + 53))
    return order_key(canon(part * (double)sc));
  double acc = 0.0;
#pragma unroll 1
  for (int v = 0; v < nvec; ++v) {
    const v4u cv = row[(long)v * kWave];   // the same address in every lane
    double x[16];
    widen(cv, x, uint8_t());
#pragma unroll
    for (int e = 0; e < 16; ++e) acc = fma((double)__uint_as_float((uint32_t)hl[16 * v + e] << 16), x[e], acc);
  }
  return order_key(canon(acc * (double)sc));
}

// Canonical keys of this thread's centroids first + i for the bits i of
// `mask`: the float64 chain over k in order from +0.0 (every product exact),
// rounded once to fp32; the masked chains run interleaved, with 16 vectors
// in flight.  For recomputing a whole row.
template <int EPT>
__device__ __forceinline__ void canonical_keys(uint32_t (&key)[EPT], uint32_t mask, int first,
                                               const uint16_t* hrow, const v4u* __restrict__ CT,
                                               int d) {
  if (!mask) return;
  const int nvec = d / 8;
  const v4u* base = CT + (long)(first / kTileTokens) * nvec * kWave + (first % kTileTokens);
  double acc[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) acc[i] = 0.0;
  // 16 vectors in flight per thread (64 VGPRs); nvec is a multiple of 8
  constexpr int kAhead = EPT >= 16 ? 1 : EPT >= 8 ? 2 : EPT >= 4 ? 4 : 8;
  for (int v0 = 0; v0 < nvec; v0 += kAhead) {
    v4u w[EPT][kAhead];
#pragma unroll
    for (int i = 0; i < EPT; ++i)
#pragma unroll
      for (int u = 0; u < kAhead; ++u)
        if (mask & (1u << i)) w[i][u] = base[(long)(v0 + u) * kWave + i];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const v4u hv = *reinterpret_cast<const v4u*>(hrow + 8 * (v0 + u));
      double hx[8];
      widen(hv, hx, uint16_t());
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        if (mask & (1u << i)) {
          double x[8];
          widen(w[i][u], x, uint16_t());
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i] = fma(hx[j], x[j], acc[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i)
    if (mask & (1u << i)) key[i] = order_key(canon(acc[i]));
}

constexpr int kRepairCap = 512;   // band keys recomputed in one row (else the whole row)

// One workgroup of kTopkThreads (8 waves) per row; thread t holds centroids
// [t*EPT, t*EPT+EPT), so thread order is id order.  The K-th largest value
// of a set is the smallest of its values with fewer than K values strictly
// above it, so it can be found by counting in parallel, without a serial
// chain of steps:
//  1. Threshold: each wave finds the Kw-th largest mu_w of its 64 thread
//     maxima, Kw = ceil(K / 8) <= 64, by such counts.  Each wave then holds
//     at least Kw distinct keys >= mu_w, so the eight hold at least K keys
//     >= mu = min_w mu_w: the K-th largest key T of the row is >= mu, and
//     the top K lies among the keys >= mu (about sixty on random rows at
//     K = 32 of 2048; the K-th largest of each wave's maxima, maxed over
//     the waves, left about 140).
//  2. The keys >= mu are gathered into LDS and T is found among them: one
//     candidate per thread counted against all (up to kTopkThreads
//     candidates), else by a radix select in each wave.
//  3. One block scan of the per-thread counts of keys > T and keys == T
//     gives the number of copies of T to keep (K minus the keys above T,
//     lowest ids first), and every thread's position in the ascending id
//     list; the kept bits are assembled into the row's 64-centroid
//     selection words.
// Rows with more than kCandCap keys >= mu (K > 512 on large rows, or masses
// of equal scores) fall back to a bit-serial select over all keys with one
// barrier per bit.  K >= Nc keeps every centroid.
//
// APPROX: the scores are the matrix cores' fp32 sums S~, each within E of
// its canonical key (E = beta A (1 + 2^-8) + 2^-23 (max|S~| + beta A) +
// d 2^-125, A = |h| max_c |C_c| >= sum_k |h_k C_ck|, beta = d 2^-23: each
// instruction adds 32 exact products and the accumulator with at most 32
// roundings or truncations of fp32 precision).  With T~ the K-th largest S~,
// every centroid with S~ > T~ + 2E is in the top K (at most K - 2 others
// can reach its key) and every one with S~ < T~ - 2E is out (K centroids
// have keys above it); the band between them fills the remaining places by
// canonical keys, recomputed in this workgroup only when the band holds more
// centroids than places.  A non-finite S~ or E, more than kCandCap keys >= mu,
// or more than kRepairCap keys in the band recompute the whole row's keys
// and select on them.
template <int EPT, int MODE, bool RANK = false, bool APPROX = false>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  static_assert(EPT >= 1 && EPT <= 32 && kWave % EPT == 0, "per-thread keys");
  __shared__ __attribute__((aligned(16))) uint32_t cand[kCandCap + kCountBlock];
  __shared__ __attribute__((aligned(16))) uint32_t wmax[kTopkThreads];
  __shared__ unsigned long long words[kMaxNc / kWave];
  __shared__ uint32_t wred[kTopkWaves];
  __shared__ uint32_t part[2][kTopkWaves];
  __shared__ uint32_t scan_sh[kTopkWaves];
  __shared__ uint32_t ncand;
  extern __shared__ __attribute__((aligned(16))) unsigned char topk_dyn[];   // APPROX: h row, band list
  if ((int)blockIdx.x >= a.rows) {
    const long from = fill_split(a.fill_n);
    fill_share<kTopkThreads>(a.fill + from, a.fill_n - from, (long)blockIdx.x - a.rows,
                             (long)gridDim.x - a.rows);
    return;
  }
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int Nc = a.Nc;
  const uint32_t K = (uint32_t)a.K;
  const int first = tid * EPT;
  const float* row = a.S + (long)b * a.ldS;

  float v[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int c = first + i;
    v[i] = row[c < Nc ? c : Nc - 1];   // unconditional (clamped) loads
  }
  // APPROX: the largest centroid norm and the hidden row (into LDS, with
  // its squared norm), loaded beside the scores; the exact scores need the
  // row's squared norm only for the certified argmax
  unsigned long long cmax_bits = 0;
  double ss = 0.0;
  if (!APPROX && a.hnorm) {
#pragma unroll 1
    for (int k = tid; k < a.d; k += kTopkThreads) {
      const double f = (double)__uint_as_float((uint32_t)a.h[(long)b * a.d + k] << 16);
      ss = fma(f, f, ss);
    }
  }
  uint16_t* hrow = reinterpret_cast<uint16_t*>(topk_dyn);
  if constexpr (APPROX) {
    cmax_bits = *a.cmax;
#pragma unroll 1
    for (int k = tid; k < a.d; k += kTopkThreads) {
      const uint16_t x = a.h[(long)b * a.d + k];
      hrow[k] = x;
      const double f = (double)__uint_as_float((uint32_t)x << 16);
      ss = fma(f, f, ss);
    }
  }
  const int nwords = (Nc + kWave - 1) / kWave;
  if (MODE >= kSelMark)
    for (int w = tid; w < nwords; w += kTopkThreads) words[w] = 0ull;

  uint32_t key[EPT];
  uint32_t valid = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int c = first + i;
    pin(v[i]);
    key[i] = c < Nc ? order_key(v[i]) : 0u;
    valid |= (c < Nc ? 1u : 0u) << i;
  }

  bool exact = !APPROX;   // keys are canonical
  bool recompute = false;  // recompute every key of the row (next round)
  double E = 0.0;
  unsigned long long* band = reinterpret_cast<unsigned long long*>(topk_dyn + 2 * (size_t)a.d);
  __shared__ double dsh[kTopkWaves];
  if constexpr (APPROX) {
    // per wave: the row's squared norm, the largest |S~| and whether an S~
    // is not finite; the waves' values are combined after the first barrier
    // of the selection
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    uint32_t mx = 0, bad = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i)
      if (valid & (1u << i)) {
        const uint32_t u = __float_as_uint(v[i]) & 0x7FFFFFFFu;
        bad |= u >= 0x7F800000u ? 1u : 0u;
        mx = max(mx, u);
      }
    mx = __ockl_wfred_max_u32(mx);
    bad = __ockl_wfred_max_u32(bad);
    if (lane == 0) {
      dsh[wv] = ss;
      part[0][wv] = mx;
      part[1][wv] = bad;
    }
  }
  if (a.hnorm) {
    // the row's |h| for the certified argmax: float64 squares of the bf16
    // elements, summed (within d 2^-53 of the exact sum), rounded up
    if constexpr (!APPROX) {
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
      if (lane == 0) dsh[wv] = ss;
    }
    __syncthreads();
    if (tid == 0) {
      double t2 = 0.0;
#pragma unroll
      for (int i = 0; i < kTopkWaves; ++i) t2 += dsh[i];
      a.hnorm[b] = f32_up(sqrt(t2) * (1.0 + 0x1p-40));
    }
  }

  uint32_t sel = valid, pos = 0, tot;
  bool placed = false;   // pos already known
  const bool take_all = K >= (uint32_t)Nc;
  for (int round = 0; round < 2 && !take_all; ++round) {
    if (APPROX && recompute) {
      // the one place that recomputes a whole row's keys (rare: a
      // non-finite sum, masses of near-equal scores)
      canonical_keys<EPT>(key, valid, first, hrow, a.CT, a.d);
      exact = true;
      recompute = false;
      if (tid == 0) atomicAdd(&a.stats[1], 1ull);
    }
    // 1. threshold
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) m = max(m, key[i]);
    if (tid == 0) ncand = 0;
    wmax[tid] = m;
    __syncthreads();
    uint32_t mu = 0;
    const uint32_t Kw = (K + kTopkWaves - 1) / kTopkWaves;
    if (Kw <= (uint32_t)kWave) {
      // smallest wave maximum with fewer than Kw wave maxima above it (0, a
      // valid bound, when the wave holds fewer than Kw keys)
      const uint32_t above = count_above(wmax + wv * kWave, kWave, m);
      mu = __ockl_wfred_min_u32(above < Kw ? m : 0xFFFFFFFFu);
    }
    if (lane == 0) wred[wv] = mu;
    __syncthreads();
    mu = wred[0];
#pragma unroll
    for (int i = 1; i < kTopkWaves; ++i) mu = min(mu, wred[i]);
    if (APPROX && round == 0) {
      // E from the waves' values (published by the barriers above); a
      // non-finite S~ or E recomputes the row's keys
      double ss = 0.0;
      uint32_t mxa = 0, bada = 0;
#pragma unroll
      for (int i = 0; i < kTopkWaves; ++i) {
        ss += dsh[i];
        mxa = max(mxa, part[0][i]);
        bada |= part[1][i];
      }
      const double cmax = __longlong_as_double((long long)cmax_bits);
      const double beta = (double)a.d * 0x1p-23;
      const double A = sqrt(ss) * (1.0 + 0x1p-40) * cmax;
      E = beta * A * (1.0 + 0x1p-8) + 0x1p-23 * ((double)__uint_as_float(mxa) + beta * A) +
          (double)a.d * 0x1p-125;
      if (bada || !(E < 1e300)) {
        recompute = true;
        __syncthreads();
        continue;
      }
    }

    // 2. candidates: the keys >= mu, in any order
    uint32_t wtotal = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) wtotal += popc64(__ballot(key[i] != 0u && key[i] >= mu));
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&ncand, wtotal);
    base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const bool p = key[i] != 0u && key[i] >= mu;
      const unsigned long long pm = __ballot(p);
      const uint32_t at = base + lanes_below(pm);
      if (p && at < (uint32_t)kCandCap) cand[at] = key[i];
      base += popc64(pm);
    }
    __syncthreads();
    const int n = (int)ncand;
    if (n > kCandCap && !exact) {
      recompute = true;
      __syncthreads();
      continue;
    }
    if (n <= kCandCap) {
      uint32_t T;
      if (n <= kTopkThreads) {
        // zero the tail to a whole block (zeros are never above a key)
        if (tid < kCountBlock) cand[n + tid] = 0u;
        __syncthreads();
        const uint32_t x = tid < n ? cand[tid] : 0u;
        const uint32_t above =
            count_above(cand, (n + kCountBlock - 1) / kCountBlock * kCountBlock, x);
        const uint32_t wmin = __ockl_wfred_min_u32(x && above < K ? x : 0xFFFFFFFFu);
        if (lane == 0) wred[wv] = wmin;
        __syncthreads();
        T = wred[0];
#pragma unroll
        for (int i = 1; i < kTopkWaves; ++i) T = min(T, wred[i]);
      } else {
        uint32_t quota, copies;
        if (n <= 8 * kWave) T = cand_kth<8>(cand, n, K, &quota, &copies);
        else T = cand_kth<16>(cand, n, K, &quota, &copies);
      }
      if (!exact) {
        // 3'. the band [T~ - 2E, T~ + 2E], rounded outward to fp32 keys
        const double tv = (double)key_value(T);
        float lo = (float)(tv - 2.0 * E), hi = (float)(tv + 2.0 * E);
        if ((double)lo > tv - 2.0 * E) lo = nextafterf(lo, -__builtin_inff());
        if ((double)hi < tv + 2.0 * E) hi = nextafterf(hi, __builtin_inff());
        const uint32_t klo = order_key(lo), khi = order_key(hi);
        uint32_t gt = 0, inb = 0;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
          gt |= (key[i] > khi ? 1u : 0u) << i;
          inb |= (key[i] != 0u && key[i] >= klo && key[i] <= khi ? 1u : 0u) << i;
        }
        const uint32_t ex =
            block_excl_scan(((uint32_t)__popc(gt) << 16) | (uint32_t)__popc(inb), scan_sh, &tot);
        const uint32_t need = K - (tot >> 16), nb = tot & 0xFFFFu;
        if (nb == need) {
          // the band holds exactly the open places: no key is recomputed
          sel = gt | inb;
          pos = (ex >> 16) + (ex & 0xFFFFu);
          placed = true;
          break;
        }
        if (nb > (uint32_t)kRepairCap) {
          recompute = true;
          __syncthreads();
          continue;
        }
        // canonical keys of the band (one wave per centroid), ranked by
        // (key desc, id asc); the `need` best take the open places
        uint32_t at = ex & 0xFFFFu;
#pragma unroll
        for (int i = 0; i < EPT; ++i)
          if (inb & (1u << i)) band[at++] = (unsigned long long)(first + i);
        __syncthreads();
        for (uint32_t j = wv; j < nb; j += kTopkWaves) {
          const int c = (int)band[j];
          const uint32_t ck = wave_canonical_key(c, hrow, a.CT, a.d);
          if (lane == 0) band[j] = ((unsigned long long)ck << 32) | (0xFFFFFFFFu - (uint32_t)c);
        }
        __syncthreads();
        uint32_t keep = 0;
        at = ex & 0xFFFFu;
#pragma unroll
        for (int i = 0; i < EPT; ++i)
          if (inb & (1u << i)) {
            const unsigned long long pk = band[at++];
            uint32_t above = 0;
            for (uint32_t j = 0; j < nb; ++j) above += band[j] > pk ? 1u : 0u;
            if (above < need) keep |= 1u << i;
          }
        sel = gt | keep;
        if (tid == 0) atomicAdd(&a.stats[0], 1ull);
        break;
      }
      // 3. keys > T, then copies of T up to K in id order
      uint32_t gt = 0, eq = 0;
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        gt |= (key[i] > T ? 1u : 0u) << i;
        eq |= (key[i] == T ? 1u : 0u) << i;
      }
      const uint32_t ex =
          block_excl_scan(((uint32_t)__popc(gt) << 16) | (uint32_t)__popc(eq), scan_sh, &tot);
      const uint32_t quota = K - (tot >> 16);
      uint32_t eq_rank = ex & 0xFFFFu;
      pos = (ex >> 16) + min(eq_rank, quota);
      uint32_t keep = 0;
#pragma unroll
      for (int i = 0; i < EPT; ++i)
        if (eq & (1u << i)) {
          if (eq_rank < quota) keep |= 1u << i;
          ++eq_rank;
        }
      sel = gt | keep;
      placed = true;
    } else {
      // bit-serial over all keys: `alive` marks keys still tied with the
      // K-th largest on the bits seen so far
      uint32_t s = 0, alive = valid, kk = K;
      for (int bit = 31; bit >= 0 && kk > 0; --bit) {
        uint32_t ones = 0;
#pragma unroll
        for (int i = 0; i < EPT; ++i) ones |= ((key[i] >> bit) & 1u) << i;
        ones &= alive;
        const uint32_t wsum = __ockl_wfred_add_u32((uint32_t)__popc(ones));
        if (lane == 0) part[bit & 1][wv] = wsum;
        __syncthreads();
        uint32_t total = 0;
#pragma unroll
        for (int i = 0; i < kTopkWaves; ++i) total += part[bit & 1][i];
        if (total <= kk) {
          s |= ones;
          alive &= ~ones;
          kk -= total;
        } else {
          alive = ones;
        }
      }
      // keys still alive are equal: keep the kk lowest ids among them
      uint32_t seen = block_excl_scan((uint32_t)__popc(alive), scan_sh, &tot);
      if (kk > 0) {
#pragma unroll
        for (int i = 0; i < EPT; ++i)
          if (alive & (1u << i)) {
            if (seen < kk) s |= 1u << i;
            ++seen;
          }
      }
      sel = s;
    }
    break;
  }
  if (!placed) pos = block_excl_scan((uint32_t)__popc(sel), scan_sh, &tot);

  // outputs
  int32_t* out = a.out + (long)b * a.ldK;
#pragma unroll
  for (int i = 0; i < EPT; ++i)
    if (sel & (1u << i)) {
      if constexpr (RANK) a.rank[(long)b * a.ldR + first + i] = (int16_t)pos;
      out[pos++] = first + i;
    }

  if (MODE >= kSelMark) {
    if (take_all) __syncthreads();   // words[] cleared before any bit is set (else the rounds' barriers order it)
    if (sel) atomicOr(&words[first / kWave], (unsigned long long)sel << (first % kWave));
    __syncthreads();
    for (int w = tid; w < nwords; w += kTopkThreads) a.cl_sel[(long)w * kWave + b] = words[w];
  }
  if (MODE == kSelMark && a.best && tid == 0) a.best[b] = 0ull;
  if (MODE == kSelMark && a.amax && tid < kArgSlots) a.amax[b * kArgRowStride + tid * kArgSlotStride] = 0ull;
}

// ------------------------------------------------------------------ gather

struct GatherArgs {
  const v4u* ET;                // [n_tiles][d/vec][64] packed tiles
  const void* h;
  int d;
  const unsigned long long* cl_sel;  // [ceil(Nc/64)][64] row selection words of the centroids
  int B;
  int tpc;                      // tiles per cluster when all clusters hold as many, else 0
  const int32_t* ttok;          // [n_tiles][64] token of each slot, -1 past the cluster's end
  // tpc == 0: tile t holds slots [64t, 64t+64) of every cluster in turn,
  // and the cluster of each slot (kNoCluster past the last slot)
  const uint16_t* tcl;          // [n_tiles][64]
  int split_shift;              // 2^split_shift waves per tile share its passes
  int n_tiles;
  // by row (equal clusters; small batches, or mid ones whose selected
  // tiles carry about one row each): one wave per (row, selected
  // centroid, tile of that cluster), the centroid read from the row's top-K
  const int32_t* topk;          // [B][ldK] ascending ids
  int ldK, K;
  int by_row;
  const float* escale;          // FP8 slabs: [n_tiles][64] row scales
  unsigned long long* best;     // top-m: [64] packed (segments << 32 | keys) per row
  unsigned long long* amax;     // argmax: packed (ordered logit, ~token) slots (kArgSlots per row)
  float* out;                   // forward: [B][V] output rows (already -inf)
  int V;
  int m;                        // top-m
  unsigned long long* tm_keys;  // top-m: [B][tm_cap] tile segments of keys
  unsigned long long* tm_heads; // top-m: [B][tm_segcap] each segment's first key
  int tm_cap, tm_segcap;
  // top-m with equal clusters: each (row, tile) segment has a fixed place,
  // (rank of the cluster in the row's selection) * tpc + tile in cluster,
  // so no counter is claimed; null otherwise
  const int16_t* tm_rank;       // [B][ldR]
  int ldR;
  // certified argmax (matrix-core dots): slot norms and the per-(row, tile)
  // bound records
  const float* enorm;           // [n_tiles][64] |e| of each slot (times its FP8 scale), rounded up
  v4u* crec;                    // per (row, tile): best L, its U, others' U, token and slot
  const int16_t* crank;         // padded tiling: [B][ldR] rank of each selected centroid
  const float* hnorm;           // [B] each row's |h|, rounded up (by the top-K kernel)
};

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  return __ockl_wfred_max_u64(v);
}

// Up to RB lowest rows of `mask` (taken out of it); unused slots repeat
// `fill`, a valid row, so that loads for them stay in bounds.
template <int RB>
__device__ __forceinline__ int take_rows(unsigned long long& mask, int (&rows)[RB], int fill) {
  int n = 0;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    if (mask) {
      rows[r] = __builtin_ctzll(mask);
      mask &= mask - 1ull;
      ++n;
    } else {
      rows[r] = r == 0 ? fill : rows[0];
    }
  }
  return n;
}

// Register stages of the gather's tile ring (chunks of 64 dims in flight
// per wave).  Four hold a whole 256-dim bf16 tile (212 registers, two waves
// a SIMD); fewer stages fit more waves.  Measured on the sweep head (µs per
// call; four / three / two stages): without the split (B < 48) three is
// best or level everywhere (B=16 argmax 22.2 / 21.9 / 22.8, B=32 27.6 /
// 27.3 / 28.8); with the tile's passes split over two waves (B=64, twice
// the waves) the argmax and the top-m take two (34.1 / 33.8 / 33.3 and
// 39.4 / 39.0 / 38.0), the forward, whose candidate stores share the
// waves' memory counter, four (46.1 / 46.6 / 47.3), and FP8 slabs, half the
// bytes a chunk, three (28.4 / 27.9 / 28.3).  By row (one row a wave, up
// to a few thousand waves) bf16 takes three, the same as four up to B=4 and
// 0.15-0.3 µs faster from B=8 to 32 (136 VGPRs against 168; two stages, 102
// VGPRs and four waves a SIMD, were 0.1-0.3 µs slower than three), and FP8
// four (26.1 against 26.2 µs at B=64).  fp32 chunks are twice as large:
// two.
template <typename T>
constexpr int kGatherStagesByRow = std::is_same<T, float>::value ? 2 : std::is_same<T, uint8_t>::value ? 4 : 3;
template <typename T, int MODE, bool SPLIT>
constexpr int kGatherStages = std::is_same<T, float>::value     ? 2
                              : std::is_same<T, uint8_t>::value ? 3
                              : !SPLIT                          ? 3
                              : MODE == kMasked                 ? 4
                                                                : 2;
constexpr bool kGatherStream = true;    // non-temporal slab loads (read once per call: 21.1 -> 20.1 us at B=64)

// Tile t of the tile grid: the rows that selected a cluster of the tile
// (mask) and, in each lane, the rows that selected the cluster of the
// lane's slot (lane_rows); cl is the tile's cluster in the padded tiling.
__device__ __forceinline__ void tile_rows(const GatherArgs& a, int t, unsigned long long& mask,
                                          unsigned long long& lane_rows, int& cl) {
  const int lane = threadIdx.x & (kWave - 1);
  if (a.tpc > 0) {
    const int c = t / a.tpc;
    cl = c;
    // lane b reads row b's selection word of c's 64-centroid block
    const unsigned long long word = lane < a.B ? a.cl_sel[(long)(c / kWave) * kWave + lane] : 0ull;
    mask = __ballot((word >> (c % kWave)) & 1ull);
    lane_rows = mask;
    return;
  }
  // the tile's slots belong to consecutive clusters: for each one, lane b
  // reads row b's selection word of its 64-centroid block (again only when
  // the block changes) and a ballot gives the rows that selected it
  const int myc = a.tcl[(long)t * kWave + lane];
  unsigned long long todo = __ballot(myc != kNoCluster);
  mask = 0ull;
  lane_rows = 0ull;
  int blk = -1;
  unsigned long long word = 0ull;
  while (todo) {
    const int c = __builtin_amdgcn_readlane(myc, (int)__builtin_ctzll(todo));
    if (c / kWave != blk) {
      blk = c / kWave;
      word = lane < a.B ? a.cl_sel[(long)blk * kWave + lane] : 0ull;
    }
    const unsigned long long m = __ballot((word >> (c % kWave)) & 1ull);
    const bool mine = myc == c;
    if (mine) lane_rows = m;
    mask |= m;
    todo &= ~__ballot(mine);
  }
}

// One wave per packed tile (2^split_shift waves from 48 rows), or, by row,
// one wave per selected (row, centroid, tile).  Once the rows that selected
// the tile's cluster are known, the tile, the hidden rows and the slots'
// token ids are all requested at once: they are addressed by the tile index
// alone.  With equal tile counts per cluster the cluster follows from the
// tile index too, so the selection words (by row: the row's top-K id) are
// the only load before the tile's.
template <typename T, int RB, int MODE, int NCH, int STG>
__global__ __launch_bounds__(64) void gather_kernel(GatherArgs a) {
  const int lane = threadIdx.x;
  // 2^split_shift waves per tile; the tile's passes of RB rows are dealt to
  // them in turn, so a tile many rows selected is not one long wave.  The
  // grid is slot-major (wave slot * n_tiles + t): workgroups are dealt to
  // the XCDs round-robin by index, and most tiles have a single pass, so
  // consecutive waves of one tile would leave every other XCD without work,
  // and the first slot's waves, the ones with work, are dispatched first.
  const int nsplit = 1 << a.split_shift;
  int t;
  int cl = 0;          // the tile's cluster (tile grid)
  int fixed_seg = 0;   // by row: the wave's fixed top-m segment
  unsigned long long mask;        // rows that selected a cluster of the tile, taken pass by pass
  unsigned long long lane_rows;   // rows that selected this lane's cluster
  auto skip_passes = [&](int n) {
    for (int i = 0; i < n * RB && mask; ++i) mask &= mask - 1ull;
  };
  if (a.by_row) {
    // a tile two rows selected is dotted (and read) by two waves, but no
    // wave is launched for a tile nobody selected, and the waves spread
    // evenly over the CUs
    const int per_row = a.K * a.tpc;
    const int b = (int)blockIdx.x / per_row;
    const int rem = (int)blockIdx.x - b * per_row;
    const int k = rem / a.tpc;
    t = a.topk[(long)b * a.ldK + k] * a.tpc + (rem - k * a.tpc);
    fixed_seg = rem;
    mask = 1ull << b;
    lane_rows = mask;
  } else {
    const int slot = (int)blockIdx.x / a.n_tiles;
    t = (int)blockIdx.x - slot * a.n_tiles;
    tile_rows(a, t, mask, lane_rows, cl);
    skip_passes(slot);
    if (!mask) return;   // no row selected a cluster of this tile, or no pass left for this wave
  }
  // the token ids are needed only after the first batch is dotted: they
  // are waited for there, not before the tile loads go out
  int tok = a.ttok[(long)t * kWave + lane];
  // FP8 slabs: the slot's row scale, applied to the finished chain
  float sc = 1.0f;
  if constexpr (std::is_same<T, uint8_t>::value) sc = a.escale[(long)t * kWave + lane];
  const long tile_vecs = (long)(a.d / Elem<T>::kPerVec) * kWave;
  const v4u* wt = a.ET + (long)t * tile_vecs;
  const auto* h = reinterpret_cast<const typename Elem<T>::hidden*>(a.h);

  // argmax: wave maximum of the packed (ordered logit, ~token) per row,
  // max-ed into the row's slot; forward: each candidate logit stored at its
  // token's column; top-m: the tile's 64 packed keys for the row stored as
  // one segment of the row's list, with the segment's maximum as its head
  int rk[RB];   // top-m on the tile grid: each pass row's rank of the cluster
  auto finish = [&](const int (&rows)[RB], int nrows, const double (&acc)[RB]) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (r < nrows) {
        const float f = std::is_same<T, uint8_t>::value ? canon(acc[r] * (double)sc) : canon(acc[r]);
        // a candidate: a token in a cluster this row selected
        const bool cand = tok >= 0 && ((lane_rows >> rows[r]) & 1ull);
        if (MODE == kArgmax) {
          unsigned long long k = 0ull;
          if (cand)
            k = ((unsigned long long)order_key(f) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)tok);
          k = wave_max_u64(k);
          // result unused: no stall; one of the row's slots, by wave index
          if (lane == 0)
            atomicMax(&a.amax[rows[r] * kArgRowStride + (int)(blockIdx.x % kArgSlots) * kArgSlotStride], k);
        } else if (MODE == kMasked) {
          if (cand) a.out[(long)rows[r] * a.V + tok] = f;
        } else {
          unsigned long long k = 0ull;
          if (cand)
            k = ((unsigned long long)order_key(f) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)tok);
          // the segment is the tile's 64 keys as they are (zero where the
          // slot holds no token; no key is 0) and its head the largest
          uint32_t seg, base;
          if (a.tm_rank) {
            seg = (uint32_t)(a.by_row ? fixed_seg : rk[r] * a.tpc + (t - cl * a.tpc));
            base = seg * (uint32_t)kTileTokens;
          } else {
            unsigned long long at = 0ull;
            if (lane == 0) at = atomicAdd(&a.best[rows[r]], (1ull << 32) | (unsigned long long)kTileTokens);
            seg = __builtin_amdgcn_readfirstlane((uint32_t)(at >> 32));
            base = __builtin_amdgcn_readfirstlane((uint32_t)at);
          }
          a.tm_keys[(long)rows[r] * a.tm_cap + base + lane] = k;
          const unsigned long long mx = wave_max_u64(k);
          if (lane == 0) a.tm_heads[(long)rows[r] * a.tm_segcap + seg] = mx;
        }
      }
    }
  };

  while (mask) {
    // the tile loads are invariant across batches; keep them in the loop
    // (hoisted, they would all be live at once)
    uint32_t zero = 0;
    asm volatile("" : "+s"(zero));
    const v4u* wtb = wt + zero;
    int rows[RB];
    const int nrows = take_rows<RB>(mask, rows, 0);
    if constexpr (MODE == kTopM) {
      // issued before the tile loads, so waiting for the first stage covers
      // them; unconditional (unused slots repeat a selecting row, and
      // without a table the load reads the row's own counter)
      const int16_t* rp = a.tm_rank ? a.tm_rank : reinterpret_cast<const int16_t*>(a.best);
#pragma unroll
      for (int r = 0; r < RB; ++r)
        rk[r] = rp[a.tm_rank && !a.by_row ? (long)rows[r] * a.ldR + cl : 0];
    }
    // lanes whose cluster none of the pass's rows selected fetch nothing
    unsigned long long prow = 0ull;
#pragma unroll
    for (int r = 0; r < RB; ++r)
      if (r < nrows) prow |= 1ull << rows[r];
    const uint32_t lane_off = ((lane_rows & prow) ? 0u : kBufRange) + 16u * (uint32_t)lane;
    double acc[RB];
    dot_tile<T, RB, NCH, STG, false, NoOp, kGatherStream, true>(wtb, a.d, h, rows, nrows,
                                                                             acc, NoOp(), lane_off);
    pin(tok);   // keep the loads out of the branches below
    pin(sc);
    finish(rows, nrows, acc);
    skip_passes(nsplit - 1);
  }
}

// ------------------------------------------------------------------ certified argmax

// Bound of a matrix-core dot: the canonical key of a (token, row) pair, as a
// real, lies within E of the fp32 result l~ (bf16 x bf16, or bf16 x decoded
// E4M3 codes, then times the slot's scale), where
// E = beta A (1 + 2^-8) + 2^-21 (|l~| + beta A) + d 2^-125, A = |h| |e| >=
// sum_k |h_k e_k| and beta = d 2^-23: every instruction adds 32 exact
// products and the accumulator with at most 32 roundings of fp32
// precision; the key's own rounding is within 2^-24 of its magnitude, the
// float64 chain within d 2^-53 of the exact sum, and the slack covers the
// fp32 arithmetic of E, l~ - E and l~ + E.
__device__ __forceinline__ float cert_bound(float lt, float A, float beta, float tiny) {
  const float bA = beta * A;
  return bA * (1.0f + 0x1p-8f) + 0x1p-21f * (fabsf(lt) + bA) + tiny;
}

// The argmax gather by matrix cores.  One wave per tile of the tile grid
// (2^split_shift waves share its passes); a pass takes up to 16 RG of the
// rows that selected a cluster of the tile, in RG groups of 16, lane r's
// row of group g the (16 g + r)-th, and every block of the tile it loads
// feeds the RG groups' instructions, so a tile that up to 16 RG rows
// selected streams from memory once.  The
// tile streams in blocks of 32 hidden dims: lane 16q + r loads the 16-byte
// vector 4kb + q of token 16m + r for each block m of 16 tokens (FP8: the
// half vector of codes, decoded to bf16), which is the A operand of
// v_mfma_f32_16x16x32_bf16 as it stands, and the B operand of group g is
// its hidden row r's dims 32kb + 8q .. +7; lane l ends with the sums of
// tokens 16m + 4(l/16) + i and row l%16 of each group.  Tokens that no row
// of the pass selected load nothing.
//
// Each (token, row) sum gets the bound E of cert_bound (|h| from the top-K
// kernel, |e| from the slot table): its canonical key lies in [L, U] =
// [l~ - E, l~ + E].  For each of its rows the wave writes one record, with
// no atomics: the largest L among the tile's candidates, that token's U,
// the largest U of the tile's other candidates, and the token and its slot
// ((token << 7) | (non-finite << 6) | slot).  The record's place is fixed
// (padded tiling: the cluster's rank in the row's selection times tpc plus
// the tile in the cluster, so a row's records are contiguous; contiguous
// tiling: the tile).  Every (row, tile) pair of a row's selected clusters
// is written by exactly one wave, so the records need no clearing.
// The record of one row of a pass for tile t (see gather_cert_kernel):
// this lane's best candidate for the row (largest L, then lowest slot), its
// U and the largest U of its other candidates, merged over the row's four
// lanes (xor 16, then 32) and written by the first.  acc holds the lane's
// sums of tokens 16m + 4(lane/16) + i for the row.
template <bool F8>
__device__ __forceinline__ void cert_record(const GatherArgs& a, const v4f (&acc)[4], int myrow, float hn,
                                            const v4u (&tok4)[4], const v4u (&en4)[4],
                                            const v4u (&sc4)[4], const unsigned long long* lr,
                                            int t, int cl, long tb, float beta, float tiny) {
  const int kq = (threadIdx.x & (kWave - 1)) >> 4;
  uint32_t bl = 0u, bu = 0u, u2 = 0u, btau = 0u, bad = 0u;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tau = 16 * m + 4 * kq + i;
      const int tok = (int)tok4[m][i];
      float lt = acc[m][i];
      if constexpr (F8) lt *= __uint_as_float(sc4[m][i]);
      const float E = cert_bound(lt, hn * __uint_as_float(en4[m][i]), beta, tiny);
      if (myrow >= 0 && tok >= 0 && ((lr[tau] >> myrow) & 1ull)) {
        // fails for a NaN too
        if (!(fabsf(lt) <= 0x1.fffffep127f && E <= 0x1.fffffep127f)) bad = 1u;
        const uint32_t lk = order_key(lt - E), uk = order_key(lt + E);
        if (lk > bl) {   // slots rise with i, so a tie keeps the lower one
          u2 = max(u2, bu);
          bl = lk;
          bu = uk;
          btau = (uint32_t)tau;
        } else {
          u2 = max(u2, uk);
        }
      }
    }
  }
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    const uint32_t obl = (uint32_t)__shfl_xor((int)bl, o), obu = (uint32_t)__shfl_xor((int)bu, o);
    const uint32_t ou2 = (uint32_t)__shfl_xor((int)u2, o), otau = (uint32_t)__shfl_xor((int)btau, o);
    bad |= (uint32_t)__shfl_xor((int)bad, o);
    const bool take = obl > bl || (obl == bl && otau < btau);
    u2 = max(max(u2, ou2), take ? bu : obu);
    if (take) {
      bl = obl;
      bu = obu;
      btau = otau;
    }
  }
  if (kq == 0 && myrow >= 0) {
    // padded tiling: the row's record sits at (rank of the cluster in the
    // row's selection) * tpc + tile in cluster; contiguous: at the tile
    const long at = a.tpc > 0 ? (long)myrow * a.K * a.tpc +
                                    (long)a.crank[(long)myrow * a.ldR + cl] * a.tpc + (t - cl * a.tpc)
                              : (long)myrow * a.n_tiles + t;
    // the token again from the tile's row of ids (read at the start, so a
    // cache hit), rather than sixteen ids held through the stream
    const uint32_t btok = (uint32_t)a.ttok[tb + btau];
    a.crec[at] = v4u{bl, bu, u2, (btok << 7) | (bad << 6) | btau};
  }
}

template <typename T, int NKB, int RG>
__global__ __launch_bounds__(64) void gather_cert_kernel(GatherArgs a) {
  constexpr bool F8 = std::is_same<T, uint8_t>::value;
  static_assert(F8 || std::is_same<T, uint16_t>::value, "bf16 or E4M3 slabs");
  static_assert(RG == 1 || RG == 2 || RG == 4, "row groups per pass");
  constexpr int PR = 16 * RG;                    // rows per pass
  __shared__ unsigned long long lr_sh[kWave];   // lane_rows of each slot of the tile
  const int lane = threadIdx.x;
  const int r = lane & 15, kq = lane >> 4;
  const int nsplit = 1 << a.split_shift;
  const int slot = (int)blockIdx.x / a.n_tiles;
  const int t = (int)blockIdx.x - slot * a.n_tiles;
  unsigned long long mask, lane_rows;
  int cl = 0;
  tile_rows(a, t, mask, lane_rows, cl);
  for (int i = 0; i < PR * slot && mask; ++i) mask &= mask - 1ull;
  if (!mask) return;
  lr_sh[lane] = lane_rows;
  const long tb = (long)t * kWave;
  // the tokens, norms (and scales) of this lane's sixteen outputs
  v4u tok4[4], en4[4], sc4[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const long o = tb + 16 * m + 4 * kq;
    tok4[m] = *reinterpret_cast<const v4u*>(a.ttok + o);
    en4[m] = *reinterpret_cast<const v4u*>(a.enorm + o);
    if constexpr (F8) sc4[m] = *reinterpret_cast<const v4u*>(a.escale + o);
  }
  __syncthreads();
  const int d = a.d;
  const int nkb = NKB > 0 ? NKB : d / 32;
  const float beta = (float)d * 0x1p-23f;
  const float tiny = (float)d * 0x1p-125f;
  const v4u* wt = a.ET + tb * (d / Elem<T>::kPerVec);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<v4u*>(wt), (short)0, (int)kBufRange, (int)kBufWord3);
  const auto* hb = reinterpret_cast<const uint16_t*>(a.h);

  while (mask) {
    // this pass's rows: lane r of group g takes the (16 g + r)-th lowest bit
    // of mask
    int myrow[RG];
    unsigned long long prow = 0ull;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      myrow[g] = -1;
      for (int i = 0; i < 16 && mask; ++i) {
        const int b = __builtin_ctzll(mask);
        mask &= mask - 1ull;
        if (r == i) myrow[g] = b;
        prow |= 1ull << b;
      }
    }
    for (int i = 0; i < PR * (nsplit - 1) && mask; ++i) mask &= mask - 1ull;
    uint32_t aoff[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int tau = 16 * m + r;
      const bool act = (lr_sh[tau] & prow) != 0ull;
      aoff[m] = (act ? 0u : kBufRange) + 16u * (uint32_t)tau + (F8 ? 8u * (uint32_t)(kq & 1) : 0u);
    }
    const v4u* hp[RG];
    float hn[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      // a valid row for every lane
      const int hrow = myrow[g] >= 0 ? myrow[g] : (int)__builtin_ctzll(prow);
      hp[g] = reinterpret_cast<const v4u*>(hb + (long)hrow * d) + kq;
      hn[g] = a.hnorm[hrow];
    }

    v4f acc[RG][4];
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[g][m] = v4f{0.f, 0.f, 0.f, 0.f};
    // groups of G blocks in two register stages, loads clamped to the last
    // block (so unconditional) and the blocks past the end skipped; with
    // four row groups each block's hidden vectors take as many registers as
    // its tile vectors, so the stages hold half the blocks
    constexpr int G = RG >= 4 ? 2 : 4;
    using AT = typename std::conditional<F8, v2u, v4u>::type;
    struct Stage {
      AT x[G][4];
      v4u h[G][RG];
    };
    auto load = [&](Stage& st, int k0) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int kb = min(k0 + j, nkb - 1);
        // vector of this lane's dims: bf16 4kb + q, E4M3 2kb + q/2 (half q%2)
        const uint32_t voff = (uint32_t)((F8 ? 2 * kb + (kq >> 1) : 4 * kb + kq) * kWave * 16);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if constexpr (F8) st.x[j][m] = __builtin_amdgcn_raw_buffer_load_b64(rsrc, aoff[m] + voff, 0, 2);
          else st.x[j][m] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, aoff[m] + voff, 0, 2);
        }
#pragma unroll
        for (int g = 0; g < RG; ++g) st.h[j][g] = hp[g][4 * kb];
      }
    };
    auto run = [&](const Stage& st, int k0) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (k0 + j < nkb) {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            v4u av;
            if constexpr (F8) {
              // E4M3 -> fp32 exactly, then the upper halves: exact bf16
#pragma unroll
              for (int w = 0; w < 2; ++w) {
                const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)st.x[j][m][w], false);
                const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)st.x[j][m][w], true);
                av[2 * w] = (__float_as_uint(lo.x) >> 16) | (__float_as_uint(lo.y) & 0xFFFF0000u);
                av[2 * w + 1] = (__float_as_uint(hi.x) >> 16) | (__float_as_uint(hi.y) & 0xFFFF0000u);
              }
            } else {
              av = st.x[j][m];
            }
#pragma unroll
            for (int g = 0; g < RG; ++g)
              acc[g][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av),
                                                                  __builtin_bit_cast(v8bf, st.h[j][g]),
                                                                  acc[g][m], 0, 0, 0);
          }
        }
      }
    };
    Stage st0, st1;
    load(st0, 0);
    if (nkb > G) load(st1, G);
#pragma unroll
    for (int k0 = 0; k0 < nkb; k0 += 2 * G) {
      run(st0, k0);
      if (k0 + 2 * G < nkb) load(st0, k0 + 2 * G);
      if (k0 + G < nkb) {
        run(st1, k0 + G);
        if (k0 + 3 * G < nkb) load(st1, k0 + 3 * G);
      }
    }

#pragma unroll
    for (int g = 0; g < RG; ++g)
      cert_record<F8>(a, acc[g], myrow[g], hn[g], tok4, en4, sc4, lr_sh, t, cl, tb, beta, tiny);
  }
}

// The certified gather for passes of 64 rows in four groups (selected tiles
// carrying more than 32 rows on average, d <= kCertHlMaxD).  The pass's
// hidden rows sit in LDS, loaded once per workgroup, each row padded by 16
// bytes so that the 16 rows an instruction's B operand reads fall in
// different banks; a wave's register stages then hold tile blocks only,
// twice as many as when each block's hidden vectors ride along.  The grid
// is persistent: kCertHlWaves waves a workgroup, one workgroup a CU (the
// rows take most of its LDS), each wave taking tiles in turn; every wave
// leaves after its last tile.
constexpr int kCertHlWaves = 8;
constexpr int kCertHlMaxD = 1024;
constexpr int kCertHlGroups = 256;

template <typename T, int NKB>
__global__ __launch_bounds__(64 * kCertHlWaves) void gather_cert_hl_kernel(GatherArgs a) {
  constexpr bool F8 = std::is_same<T, uint8_t>::value;
  static_assert(F8 || std::is_same<T, uint16_t>::value, "bf16 or E4M3 slabs");
  extern __shared__ __attribute__((aligned(16))) unsigned char hl_dyn[];   // [B][2d + 16] bytes
  // per wave, for the tile at hand: each slot's rows (lane_rows), token,
  // |e| and FP8 scale; the last three wait in LDS while the tile streams
  __shared__ unsigned long long lr_all[kCertHlWaves][kWave];
  __shared__ __attribute__((aligned(16))) uint32_t tok_all[kCertHlWaves][kWave];
  __shared__ __attribute__((aligned(16))) uint32_t en_all[kCertHlWaves][kWave];
  __shared__ __attribute__((aligned(16))) uint32_t sc_all[F8 ? kCertHlWaves : 1][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = (int)threadIdx.x / kWave;
  const int r = lane & 15, kq = lane >> 4;
  const int d = a.d;
  const int nkb = NKB > 0 ? NKB : d / 32;
  const int ldh = 2 * d + 16;
  {
    const int nv = d / 8;   // 16-byte vectors a row
    const v4u* hsrc = static_cast<const v4u*>(a.h);
    for (int i = threadIdx.x; i < a.B * nv; i += (int)blockDim.x) {
      const int b = i / nv, v = i - b * nv;
      *reinterpret_cast<v4u*>(hl_dyn + (long)b * ldh + 16 * v) = hsrc[(long)b * nv + v];
    }
  }
  __syncthreads();
  unsigned long long* lr = lr_all[wv];
  const float beta = (float)d * 0x1p-23f;
  const float tiny = (float)d * 0x1p-125f;
  for (int t = (int)blockIdx.x * kCertHlWaves + wv; t < a.n_tiles; t += (int)gridDim.x * kCertHlWaves) {
    unsigned long long mask, lane_rows;
    int cl = 0;
    tile_rows(a, t, mask, lane_rows, cl);
    if (!mask) continue;
    // the previous tile's reads of lr are done before this write (one wave:
    // its LDS operations run in order; the fences keep the compiler's too)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    lr[lane] = lane_rows;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const long tb = (long)t * kWave;
    // this lane's slot: loaded now, put in LDS once the first blocks' loads
    // are on their way
    const uint32_t my_tok = (uint32_t)a.ttok[tb + lane];
    const uint32_t my_en = __float_as_uint(a.enorm[tb + lane]);
    uint32_t my_sc = 0u;
    if constexpr (F8) my_sc = __float_as_uint(a.escale[tb + lane]);
    const v4u* wt = a.ET + tb * (d / Elem<T>::kPerVec);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<v4u*>(wt), (short)0, (int)kBufRange, (int)kBufWord3);
    // the pass: lane r of group g takes the (16 g + r)-th row of mask (at
    // most 64 rows: one pass)
    int myrow[4];
    unsigned long long prow = 0ull;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      myrow[g] = -1;
      for (int i = 0; i < 16 && mask; ++i) {
        const int b = __builtin_ctzll(mask);
        mask &= mask - 1ull;
        if (r == i) myrow[g] = b;
        prow |= 1ull << b;
      }
    }
    uint32_t aoff[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int tau = 16 * m + r;
      const bool act = (lr[tau] & prow) != 0ull;
      aoff[m] = (act ? 0u : kBufRange) + 16u * (uint32_t)tau + (F8 ? 8u * (uint32_t)(kq & 1) : 0u);
    }
    uint32_t hoff[4];
    float hn[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int hrow = myrow[g] >= 0 ? myrow[g] : (int)__builtin_ctzll(prow);   // a valid row
      hoff[g] = (uint32_t)(hrow * ldh + 16 * kq);
      hn[g] = a.hnorm[hrow];
    }
    v4f acc[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[g][m] = v4f{0.f, 0.f, 0.f, 0.f};
    // blocks a register stage (two stages): the most that fit in the 256
    // registers a wave has at two waves a SIMD beside the 64 accumulators
    constexpr int G = 3;
    using AT = typename std::conditional<F8, v2u, v4u>::type;
    struct Stage {
      AT x[G][4];
    };
    auto load = [&](Stage& st, int k0) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int kb = min(k0 + j, nkb - 1);
        const uint32_t voff = (uint32_t)((F8 ? 2 * kb + (kq >> 1) : 4 * kb + kq) * kWave * 16);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if constexpr (F8) st.x[j][m] = __builtin_amdgcn_raw_buffer_load_b64(rsrc, aoff[m] + voff, 0, 2);
          else st.x[j][m] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, aoff[m] + voff, 0, 2);
        }
      }
    };
    auto run = [&](const Stage& st, int k0) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (k0 + j < nkb) {
          v4u hv[4];
#pragma unroll
          for (int g = 0; g < 4; ++g)
            hv[g] = *reinterpret_cast<const v4u*>(hl_dyn + hoff[g] + 64 * (k0 + j));
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            v4u av;
            if constexpr (F8) {
#pragma unroll
              for (int w = 0; w < 2; ++w) {
                const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)st.x[j][m][w], false);
                const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)st.x[j][m][w], true);
                av[2 * w] = (__float_as_uint(lo.x) >> 16) | (__float_as_uint(lo.y) & 0xFFFF0000u);
                av[2 * w + 1] = (__float_as_uint(hi.x) >> 16) | (__float_as_uint(hi.y) & 0xFFFF0000u);
              }
            } else {
              av = st.x[j][m];
            }
#pragma unroll
            for (int g = 0; g < 4; ++g)
              acc[g][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av),
                                                                  __builtin_bit_cast(v8bf, hv[g]),
                                                                  acc[g][m], 0, 0, 0);
          }
        }
      }
    };
    Stage st0, st1;
    load(st0, 0);
    if (nkb > G) load(st1, G);
    __builtin_amdgcn_sched_barrier(0);
    tok_all[wv][lane] = my_tok;
    en_all[wv][lane] = my_en;
    if constexpr (F8) sc_all[wv][lane] = my_sc;
#pragma unroll
    for (int k0 = 0; k0 < nkb; k0 += 2 * G) {
      run(st0, k0);
      if (k0 + 2 * G < nkb) load(st0, k0 + 2 * G);
      if (k0 + G < nkb) {
        run(st1, k0 + G);
        if (k0 + 3 * G < nkb) load(st1, k0 + 3 * G);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    v4u tok4[4], en4[4], sc4[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      tok4[m] = *reinterpret_cast<const v4u*>(&tok_all[wv][16 * m + 4 * kq]);
      en4[m] = *reinterpret_cast<const v4u*>(&en_all[wv][16 * m + 4 * kq]);
      if constexpr (F8) sc4[m] = *reinterpret_cast<const v4u*>(&sc_all[wv][16 * m + 4 * kq]);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
      cert_record<F8>(a, acc[g], myrow[g], hn[g], tok4, en4, sc4, lr, t, cl, tb, beta, tiny);
  }
}

// The canonical key of one slot by one thread: the float64 chain over the
// hidden dims in order (FP8: times the slot's scale), for a whole recompute.
template <typename T>
__device__ uint32_t slot_chain_key(const v4u* __restrict__ row, const uint16_t* hl, int d, float sc) {
  constexpr int PV = Elem<T>::kPerVec;
  double acc = 0.0;
#pragma unroll 1
  for (int v = 0; v < d / PV; ++v) {
    double x[PV];
    widen(row[(long)v * kWave], x, T());
#pragma unroll
    for (int e = 0; e < PV; ++e) acc = fma((double)__uint_as_float((uint32_t)hl[PV * v + e] << 16), x[e], acc);
  }
  return order_key(canon(std::is_same<T, uint8_t>::value ? acc * (double)sc : acc));
}

struct CertArgs {
  const v4u* crec;        // [B][n_tiles] records of the gather
  int n_tiles;
  const v4u* ET;
  const float* escale;
  const int32_t* ttok;
  const uint16_t* tcl;    // contiguous tiling: cluster of each slot
  const unsigned long long* cl_sel;
  const uint16_t* h;      // [B][d] bf16
  int d;
  // the row's selected clusters and their tiles
  const int32_t* topk;
  int ldK, K;
  const int32_t* offsets;
  int tpc;
  int32_t* tokens;
};
constexpr int kCertThreads = 256;
constexpr int kCertWaves = kCertThreads / kWave;
constexpr int kSurvCap = 128;   // tokens, and whole tiles, recomputed by waves (more: the whole row)

// The k-th selected cluster of row b and its tiles [t0, t1) in the tiling;
// a contiguous tile shared with the previous selected cluster is left to it.
__device__ __forceinline__ void cert_tiles(const CertArgs& f, int b, int k, int& c, long& t0, long& t1) {
  c = f.topk[(long)b * f.ldK + k];
  const int lo = f.offsets[c], hi = f.offsets[c + 1];
  if (f.tpc > 0) {
    t0 = (long)c * f.tpc;
    t1 = t0 + f.tpc;
    return;
  }
  t0 = lo / kWave;
  t1 = hi > lo ? (long)(hi - 1) / kWave + 1 : t0;
  if (k > 0 && t1 > t0) {
    const int pc = f.topk[(long)b * f.ldK + k - 1];
    const int phi = f.offsets[pc + 1], plo = f.offsets[pc];
    if (phi > plo && (phi - 1) / kWave == t0) ++t0;
  }
}

// fn(t) for every tile of row b's selected clusters, spread over the
// workgroup: per 256 clusters, a scan of their tile counts, then thread i
// takes the tiles i, i + 256, ... of the run (found by binary search).  A
// tile shared by two selected clusters with an empty one between them comes
// twice, which the callers allow.  Every thread of the block must call it.
template <typename F>
__device__ __forceinline__ void for_row_tiles(const CertArgs& f, int b, uint32_t* pre_sh, long* t0_sh,
                                              uint32_t* scan_sh, F&& fn) {
  const int tid = threadIdx.x;
  for (int k0 = 0; k0 < f.K; k0 += kCertThreads) {
    const int k = k0 + tid;
    int c = 0;
    long t0 = 0, t1 = 0;
    if (k < f.K) cert_tiles(f, b, k, c, t0, t1);
    uint32_t tot;
    const uint32_t pre = block_excl_scan<kCertWaves>((uint32_t)(t1 - t0), scan_sh, &tot);
    pre_sh[tid] = pre;
    t0_sh[tid] = t0;
    __syncthreads();
    const int last = min(kCertThreads, f.K - k0) - 1;
    for (uint32_t i = tid; i < tot; i += kCertThreads) {
      // the last cluster whose run starts at or before i (empty ones share
      // the next one's start and are passed over)
      int lo = 0, hi = last;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre_sh[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      fn(t0_sh[lo] + (long)(i - pre_sh[lo]));
    }
    __syncthreads();
  }
}

// One workgroup per row.  M, the largest L over the row's records, is a
// lower bound of the row's best canonical key; a token can win only if its
// U reaches M.  The records name each tile's best token (with its U) and
// bound its other candidates' U: when only one named token reaches M and
// no tile's others can, that token wins outright, with no other load (the
// usual case; on the padded tiling the row's records are one contiguous
// run, read once).  Otherwise the hidden row goes to LDS, the named tokens
// that reach M get canonical keys (a wave each, by the exact-sum test) and
// the tiles whose others can reach M are recomputed whole (a lane per
// slot); past kSurvCap of either, or with a non-finite record, every
// candidate of the row is recomputed (a thread per slot).  The row's token
// is the largest (key, ~token); -1 with no candidate.
template <typename T>
__global__ __launch_bounds__(kCertThreads) void finalize_cert_kernel(CertArgs f) {
  constexpr bool F8 = std::is_same<T, uint8_t>::value;
  constexpr int PV = Elem<T>::kPerVec;
  constexpr int R = 4;   // records a thread holds from the first pass to the second
  extern __shared__ __attribute__((aligned(16))) unsigned char cert_dyn[];
  uint16_t* hrow = reinterpret_cast<uint16_t*>(cert_dyn);   // [d]
  __shared__ uint32_t surv[kSurvCap];      // (record << 6) | slot of named tokens that reach M
  __shared__ uint32_t fullt[kSurvCap];     // records whose tile's other candidates reach M
  __shared__ unsigned long long wbest[kCertWaves];
  __shared__ uint32_t wM[kCertWaves];
  __shared__ uint32_t nsurv, nfull, nbad, tok0;
  __shared__ uint32_t tile_pre[kCertThreads];
  __shared__ long tile_t0[kCertThreads];
  __shared__ uint32_t scan_sh[kCertWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int d = f.d;
  const bool padded = f.tpc > 0;
  const int nrec = padded ? f.K * f.tpc : 0;
  const v4u* prec = f.crec + (long)b * nrec;         // padded: the row's records in order
  const v4u* trec = f.crec + (long)b * f.n_tiles;    // contiguous: by tile
  if (tid == 0) {
    nsurv = 0u;
    nfull = 0u;
    nbad = 0u;
  }
  // the tile of record i (padded), or the tile itself (contiguous)
  auto tile_of = [&](uint32_t i) -> long {
    return padded ? (long)f.topk[(long)b * f.ldK + (int)(i / (uint32_t)f.tpc)] * f.tpc + (long)(i % (uint32_t)f.tpc)
                  : (long)i;
  };
  v4u cache[R];
  uint32_t M = 0u, bad = 0u;
  if (padded) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int i = tid + kCertThreads * j;
      cache[j] = i < nrec ? prec[i] : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      M = max(M, cache[j][0]);
      bad |= (cache[j][3] >> 6) & 1u;
    }
    for (int i = tid + kCertThreads * R; i < nrec; i += kCertThreads) {
      const v4u rc = prec[i];
      M = max(M, rc[0]);
      bad |= (rc[3] >> 6) & 1u;
    }
  } else {
    for_row_tiles(f, b, tile_pre, tile_t0, scan_sh, [&](long t) {
      const v4u rc = trec[t];
      M = max(M, rc[0]);
      bad |= (rc[3] >> 6) & 1u;
    });
  }
  M = __ockl_wfred_max_u32(M);
  bad = __ockl_wfred_max_u32(bad);
  if (lane == 0) {
    wM[wv] = M;
    if (bad) nbad = 1u;
  }
  __syncthreads();
  M = wM[0];
#pragma unroll
  for (int i = 1; i < kCertWaves; ++i) M = max(M, wM[i]);
  bool whole = nbad != 0u;
  // the named tokens and the tiles that can reach M
  auto consider = [&](const v4u& rc, uint32_t i) {
    if (rc[1] >= M) {
      const uint32_t at = atomicAdd(&nsurv, 1u);
      if (at < (uint32_t)kSurvCap) surv[at] = (i << 6) | (rc[3] & 63u);
      if (at == 0u) tok0 = rc[3] >> 7;
    }
    if (rc[2] >= M) {
      const uint32_t at = atomicAdd(&nfull, 1u);
      if (at < (uint32_t)kSurvCap) fullt[at] = i;
    }
  };
  if (!whole) {
    if (padded) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const int i = tid + kCertThreads * j;
        if (i < nrec) consider(cache[j], (uint32_t)i);
      }
      for (int i = tid + kCertThreads * R; i < nrec; i += kCertThreads) consider(prec[i], (uint32_t)i);
    } else {
      for_row_tiles(f, b, tile_pre, tile_t0, scan_sh, [&](long t) { consider(trec[t], (uint32_t)t); });
    }
  }
  __syncthreads();
  const uint32_t ns = nsurv, nf = nfull;
  whole = whole || ns > (uint32_t)kSurvCap || nf > (uint32_t)kSurvCap;
  unsigned long long best = 0ull;
  if (!whole && ns == 1u && nf == 0u) {
    // one token can reach the best lower bound: it wins
    best = (1ull << 32) | (unsigned long long)(0xFFFFFFFFu - tok0);
  } else if (ns > 0u || whole) {
    for (int k = tid; k < d; k += kCertThreads) hrow[k] = f.h[(long)b * d + k];
    __syncthreads();
    if (!whole) {
      for (uint32_t i = wv; i < ns; i += kCertWaves) {
        const uint32_t w = surv[i];
        const long t = tile_of(w >> 6);
        const int tau = (int)(w & 63u);
        const v4u* row = f.ET + t * (d / PV) * kWave + tau;
        const uint32_t tok = (uint32_t)f.ttok[t * kWave + tau];
        const uint32_t key = F8 ? wave_row_key_fp8(row, hrow, d, f.escale[t * kWave + tau])
                                : wave_row_key(row, hrow, d);
        best = max(best, ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - tok));
      }
      // whole tiles: a lane per slot, the candidates of this row only
      for (uint32_t i = wv; i < nf; i += kCertWaves) {
        const long t = tile_of(fullt[i]);
        const int tok = f.ttok[t * kWave + lane];
        bool cand = tok >= 0;
        if (cand && !padded) {
          const int c = f.tcl[t * kWave + lane];
          cand = ((f.cl_sel[(long)(c / kWave) * kWave + b] >> (c % kWave)) & 1ull) != 0ull;
        }
        if (cand) {
          const v4u* row = f.ET + t * (d / PV) * kWave + lane;
          const uint32_t key = slot_chain_key<T>(row, hrow, d, F8 ? f.escale[t * kWave + lane] : 1.0f);
          best = max(best, ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)tok));
        }
      }
    } else {
      // every candidate of the row, a thread per slot: the float64 chain in order
      for (int k = 0; k < f.K; ++k) {
        const int c = f.topk[(long)b * f.ldK + k];
        const int lo = f.offsets[c], hi = f.offsets[c + 1];
        for (int s2 = lo + tid; s2 < hi; s2 += kCertThreads) {
          const long t = padded ? (long)c * f.tpc + (s2 - lo) / kWave : s2 / kWave;
          const int tau = padded ? (s2 - lo) % kWave : s2 % kWave;
          const v4u* row = f.ET + t * (d / PV) * kWave + tau;
          const uint32_t tok = (uint32_t)f.ttok[t * kWave + tau];
          const uint32_t key = slot_chain_key<T>(row, hrow, d, F8 ? f.escale[t * kWave + tau] : 1.0f);
          best = max(best, ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - tok));
        }
      }
    }
  }
  best = wave_max_u64(best);
  if (lane == 0) wbest[wv] = best;
  __syncthreads();
  if (tid == 0) {
    unsigned long long m = wbest[0];
#pragma unroll
    for (int i = 1; i < kCertWaves; ++i) m = max(m, wbest[i]);
    f.tokens[b] = m ? (int32_t)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFull)) : -1;
  }
}

// Slot norms for the certified argmax: |e| of each packed slot (FP8: the
// decoded codes' norm times the row scale), float64 then rounded up.
template <typename T>
__global__ __launch_bounds__(256) void slot_norm_kernel(const v4u* __restrict__ ET, const float* __restrict__ escale,
                                                        long n_slots, int d, float* __restrict__ out) {
  constexpr int PV = Elem<T>::kPerVec;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long o = (long)blockIdx.x * blockDim.x + threadIdx.x; o < n_slots; o += stride) {
    const long t = o / kWave;
    const int tau = (int)(o % kWave);
    const v4u* row = ET + t * (d / PV) * kWave + tau;
    double ss = 0.0;
    for (int v = 0; v < d / PV; ++v) {
      double x[PV];
      widen(row[(long)v * kWave], x, T());
#pragma unroll
      for (int e = 0; e < PV; ++e) ss = fma(x[e], x[e], ss);
    }
    double nrm = sqrt(ss) * (1.0 + 0x1p-40);
    if (std::is_same<T, uint8_t>::value) nrm *= (double)escale[o] * (1.0 + 0x1p-50);
    out[o] = f32_up(nrm);
  }
}

// A row's packed (ordered logit, ~token) maximum over its argmax slots.
__device__ __forceinline__ unsigned long long row_best(const unsigned long long* __restrict__ amax, int b) {
  unsigned long long v[kArgSlots];
#pragma unroll
  for (int s = 0; s < kArgSlots; ++s) v[s] = amax[b * kArgRowStride + s * kArgSlotStride];
  unsigned long long m = v[0];
#pragma unroll
  for (int s = 1; s < kArgSlots; ++s) m = max(m, v[s]);
  return m;
}

// Decode each row's packed (ordered logit, ~token) maximum; 0 means no
// candidate at all.
__global__ __launch_bounds__(64) void finalize_kernel(const unsigned long long* __restrict__ amax,
                                                      int B, int32_t* __restrict__ tokens) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) {
    const unsigned long long v = row_best(amax, b);
    tokens[b] = v ? (int32_t)(0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFull)) : -1;
  }
}

// Finalize plus the next step's input embedding: one workgroup per row
// decodes the row's token and writes emb[b] = table[token] * normalizer
// (float32 product, then the head's element type; zeros without a token).
struct EmbedArgs {
  const void* table;   // [V][dim] head dtype, indexed by token id
  int dim;             // elements per row, 16-byte rows
  float normalizer;
  void* out;           // [B][dim]
};
constexpr int kEmbedThreads = 256;

__device__ __forceinline__ v4u scale_vec(v4u v, float n, uint16_t) {
  v4u o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = bf16_rne(__uint_as_float(v[i] << 16) * n);
    const uint32_t hi = bf16_rne(__uint_as_float(v[i] & 0xFFFF0000u) * n);
    o[i] = lo | (hi << 16);
  }
  return o;
}
__device__ __forceinline__ v4u scale_vec(v4u v, float n, float) {
  v4u o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(__uint_as_float(v[i]) * n);
  return o;
}

template <typename T>
__global__ __launch_bounds__(kEmbedThreads) void finalize_embed_kernel(
    const unsigned long long* __restrict__ amax, int32_t* __restrict__ tokens, EmbedArgs e) {
  const int b = blockIdx.x;
  const unsigned long long v = row_best(amax, b);
  const int tok = v ? (int)(0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFull)) : -1;
  if (threadIdx.x == 0) tokens[b] = tok;
  const int nvec = e.dim / Elem<T>::kPerVec;
  v4u* dst = static_cast<v4u*>(e.out) + (long)b * nvec;
  if (tok < 0) {
    for (int i = threadIdx.x; i < nvec; i += kEmbedThreads) dst[i] = v4u{0u, 0u, 0u, 0u};
    return;
  }
  const v4u* src = static_cast<const v4u*>(e.table) + (long)tok * nvec;
  for (int i = threadIdx.x; i < nvec; i += kEmbedThreads) dst[i] = scale_vec(src[i], e.normalizer, T());
}

// ------------------------------------------------------------------ top-m merge

struct TopmArgs {
  const unsigned long long* cnt;    // [B] packed (segments << 32 | keys)
  const unsigned long long* keys;   // [B][cap]
  const unsigned long long* heads;  // [B][segcap]
  int cap, segcap, m;
  int fixed_segs;                   // > 0: every row has this many segments of 64 keys (zeros pad)
  int32_t* tokens;                  // [B][m]
  float* logits;                    // [B][m] logits, or log-probabilities with log_softmax
  int log_softmax;                  // log-probabilities under the softmax over the row's candidates
};


// One workgroup of kTopkThreads per row.  Each gather segment holds one
// tile's keys for the row (zeros where a slot has no token) and its head is
// their maximum, so the m-th largest head mu is a lower bound of the row's
// m-th largest key (m heads are keys >= mu), and only the m segments whose
// heads are the m largest (heads are distinct) hold keys >= mu: at most
// m*64 candidates.  Each of those counts the candidates above it; a count
// below m is its output position.  With fewer than m segments every key is
// a candidate.
//
// log_softmax: every key of the row passes through the scan below, so the
// scan also sums T = sum of exp(l - M) in float64 over all candidates but
// the row's largest key (M its logit, the largest head), each thread in
// its order, the waves' sums combined in wave order (the same result on
// every run); each output is then (l - M) - log1p(T), rounded once.
__global__ __launch_bounds__(kTopkThreads) void topm_merge_kernel(TopmArgs a) {
  extern __shared__ unsigned long long tm_lds[];   // heads [segcap], then candidates
  __shared__ uint32_t ncand;
  __shared__ unsigned long long wred[kTopkWaves];
  __shared__ unsigned long long wtop[kTopkWaves];
  __shared__ double wsum[kTopkWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int m = a.m;
  const unsigned long long c = a.fixed_segs > 0 ? 0ull : a.cnt[b];
  const int segs = a.fixed_segs > 0 ? a.fixed_segs : (int)(c >> 32);
  const int n = a.fixed_segs > 0 ? a.fixed_segs * kTileTokens : (int)(uint32_t)c;
  // keys >= mu come from the m segments whose heads are the m largest
  // (heads are distinct), so at most m * 64 of them
  const int cap_c = m * kTileTokens;
  unsigned long long* heads = tm_lds;
  unsigned long long* cand = tm_lds + a.segcap;
  const unsigned long long* hsrc = a.heads + (long)b * a.segcap;
  const unsigned long long* ksrc = a.keys + (long)b * a.cap;
  for (int i = tid; i < segs; i += kTopkThreads) heads[i] = hsrc[i];
  if (tid == 0) ncand = 0;
  __syncthreads();

  // log_softmax: the row's largest key (0: no candidate) and its logit
  unsigned long long ktop = 0ull;
  double mtop = 0.0;
  if (a.log_softmax) {
    unsigned long long hm = 0ull;
    for (int i = tid; i < segs; i += kTopkThreads) hm = max(hm, heads[i]);
    hm = __ockl_wfred_max_u64(hm);
    if (lane == 0) wtop[wv] = hm;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTopkWaves; ++i) ktop = max(ktop, wtop[i]);
    if (ktop) mtop = (double)key_value((uint32_t)(ktop >> 32));
  }
  double tsum = 0.0;

  unsigned long long mu = 0ull;
  if (segs >= m) {
    unsigned long long low = ~0ull;
    for (int i = tid; i < segs; i += kTopkThreads) {
      const unsigned long long x = heads[i];
      int above = 0;
      for (int j = 0; j < segs; ++j) above += heads[j] > x ? 1 : 0;
      if (above < m) low = min(low, x);
    }
    low = __ockl_wfred_min_u64(low);
    if (lane == 0) wred[wv] = low;
    __syncthreads();
    mu = wred[0];
#pragma unroll
    for (int i = 1; i < kTopkWaves; ++i) mu = min(mu, wred[i]);
  }
  // eight loads in flight per thread before any is tested (clamped, so
  // unconditional; a clamped repeat of the last key is dropped by i < n)
  constexpr int kScan = 8;
  for (int i0 = 0; i0 < n; i0 += kScan * kTopkThreads) {
    unsigned long long kk[kScan];
#pragma unroll
    for (int u = 0; u < kScan; ++u) kk[u] = ksrc[min(i0 + u * kTopkThreads + tid, n - 1)];
#pragma unroll
    for (int u = 0; u < kScan; ++u) {
      const unsigned long long k = kk[u];
      const bool in = i0 + u * kTopkThreads + tid < n && k != 0ull;
      if (in && k >= mu) {
        const uint32_t at = atomicAdd(&ncand, 1u);
        if (at < (uint32_t)cap_c) cand[at] = k;
      }
      if (a.log_softmax && in && k != ktop)
        tsum += exp((double)key_value((uint32_t)(k >> 32)) - mtop);
    }
  }
  if (a.log_softmax) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) tsum += __shfl_xor(tsum, o);
    if (lane == 0) wsum[wv] = tsum;
  }
  __syncthreads();
  double lg = 0.0;
  if (a.log_softmax) {
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < kTopkWaves; ++i) t += wsum[i];
    lg = log1p(t);
  }
  const int nc = min((int)ncand, cap_c);
  int32_t* tok = a.tokens + (long)b * m;
  float* val = a.logits + (long)b * m;
  for (int i = tid; i < nc; i += kTopkThreads) {
    const unsigned long long x = cand[i];
    int above = 0;
    for (int j = 0; j < nc; ++j) above += cand[j] > x ? 1 : 0;
    if (above < m) {
      tok[above] = (int32_t)(0xFFFFFFFFu - (uint32_t)x);
      const float l = key_value((uint32_t)(x >> 32));
      val[above] = a.log_softmax ? (float)(((double)l - mtop) - lg) : l;
    }
  }
  for (int p = min(nc, m) + tid; p < m; p += kTopkThreads) {
    tok[p] = -1;
    val[p] = -__builtin_inff();
  }
}

}  // namespace

// ------------------------------------------------------------------ launchers

hipError_t launch_pack(const void* W, int dtype, int d, long n_tiles, const uint32_t* tiles,
                       const int32_t* offsets, int nrows_total, void* out, hipStream_t s) {
  const int nvec = d / (dtype == 1 ? Elem<uint16_t>::kPerVec : Elem<float>::kPerVec);
  const long n_out = n_tiles * nvec * kTileTokens;
  if (n_out == 0) return hipSuccess;
  long blocks = (n_out + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const v4u*>(W), nvec, n_out, tiles, offsets, nrows_total,
                     static_cast<v4u*>(out));
  return hipGetLastError();
}

hipError_t launch_cnorm_max(const void* C, int dtype, int Nc, int d, unsigned long long* out,
                            hipStream_t s) {
  const dim3 grid((Nc + 255) / 256);
  if (dtype == 1)
    hipLaunchKernelGGL(cnorm_max_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(C), Nc, d, out);
  else
    hipLaunchKernelGGL(cnorm_max_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(C),
                       Nc, d, out);
  return hipGetLastError();
}

hipError_t launch_pack_fp8(const void* W, int d, long n_tiles, const uint32_t* tiles,
                           const int32_t* offsets, int nrows_total, void* out, float* scale,
                           hipStream_t s) {
  const long n_rows_out = n_tiles * kTileTokens;
  if (n_rows_out == 0) return hipSuccess;
  long blocks = (n_rows_out + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const uint16_t*>(W), d, n_rows_out, tiles, offsets,
                     (long)nrows_total, static_cast<v4u*>(out), scale);
  return hipGetLastError();
}

// Fill waves of the forward's projection: about one per 64 KiB of its
// share of the output rows, at least one row of the grid, at most 1024.
static int fill_grid_rows(const PassArgs& a, int gx) {
  if (!a.fill) return 0;
  const long bytes = fill_split((long)a.B * a.V) * 4;
  const long waves = std::min<long>(1024, std::max<long>(1, bytes / 65536));
  return (int)std::max<long>(1, (waves + gx - 1) / gx);
}

// Fill workgroups of the forward's top-K launch (512 threads): about one
// per 256 KiB of the rest of the rows, at least one, at most 256.
static int fill_topk_groups(const PassArgs& a) {
  if (!a.fill) return 0;
  const long n = (long)a.B * a.V;
  const long bytes = (n - fill_split(n)) * 4;
  return (int)std::min<long>(256, std::max<long>(1, bytes / 262144));
}

template <typename T, int RB, int NCH>
static void launch_scores_n(const PassArgs& a, hipStream_t s) {
  const int gx = (a.Nc + kTileTokens - 1) / kTileTokens;
  const dim3 grid(gx, (a.B + RB - 1) / RB + fill_grid_rows(a, gx));
  NormArgs nm{a.norm_w, (double)a.norm_eps, a.h_out};
  if (a.norm_w)
    hipLaunchKernelGGL((scores_kernel<T, RB, NCH, true>), grid, dim3(64),
                       (size_t)RB * a.d * sizeof(T), s, static_cast<const v4u*>(a.t.CT), a.Nc,
                       a.d, static_cast<const T*>(a.h), a.B, a.S, a.ldS, a.fill, a.V, nm);
  else
    hipLaunchKernelGGL((scores_kernel<T, RB, NCH, false>), grid, dim3(64), 0, s,
                       static_cast<const v4u*>(a.t.CT), a.Nc, a.d, static_cast<const T*>(a.h), a.B,
                       a.S, a.ldS, a.fill, a.V, nm);
}

// Hidden sizes with a straight-line chunk pipeline; others take the generic one.
#define CE_DISPATCH_NCH(d, CALL)          \
  switch ((d) / kChunk) {                 \
    case 4: CALL(4); break;               \
    case 8: CALL(8); break;               \
    case 16: CALL(16); break;             \
    default: CALL(0); break;              \
  }

template <typename T, int RB>
static void launch_scores_t(const PassArgs& a, hipStream_t s) {
#define CE_SCORES(N) launch_scores_n<T, RB, N>(a, s)
  CE_DISPATCH_NCH(a.d, CE_SCORES)
#undef CE_SCORES
}

// One row per wave: the projection at small batches is a lone wave's fp64
// chain per SIMD, so halving each wave's rows halves the critical path
// (sweep head, µs per call: B=2 17.9 → 16.5, B=16 24.1 → 22.8, B=64 37.1 →
// 36.7).  Two rows per wave (the tile widened once for both) only for the
// forward at 48 rows or more, where the grid also holds the fill waves
// (B=64: 55.2 with one row against 54.4).
// MFMA blocks of 16 centroids per wave of the approximate projection.
constexpr int kProjMB = 1;

template <int NKS>
static void launch_proj_n(const PassArgs& a, hipStream_t s) {
  const int gx = (a.Nc + 16 * kProjMB - 1) / (16 * kProjMB);
  const dim3 grid(gx, (a.B + 15) / 16 + fill_grid_rows(a, gx));
  hipLaunchKernelGGL((proj_mfma_kernel<kProjMB, NKS>), grid, dim3(64), 0, s,
                     static_cast<const v4u*>(a.t.CT), a.Nc, a.d, static_cast<const uint16_t*>(a.h),
                     a.B, a.S, a.ldS, a.fill, a.V);
}

hipError_t launch_scores(const PassArgs& a, hipStream_t s) {
  if (a.approx) {
    switch (a.d / 32) {
      case 8: launch_proj_n<8>(a, s); break;
      case 16: launch_proj_n<16>(a, s); break;
      case 32: launch_proj_n<32>(a, s); break;
      default: launch_proj_n<0>(a, s); break;
    }
    return hipGetLastError();
  }
  const bool two = a.fill != nullptr && a.B >= 48;
  if (a.dtype == 1) {
    if (two) launch_scores_t<uint16_t, 2>(a, s); else launch_scores_t<uint16_t, 1>(a, s);
  } else {
    if (two) launch_scores_t<float, 2>(a, s); else launch_scores_t<float, 1>(a, s);
  }
  return hipGetLastError();
}

static bool cert_gather(const PassArgs& a);

template <int EPT>
static void launch_topk_ept(const TopkArgs& t, int G, int mode, bool approx, hipStream_t s) {
  // the ranks (top-m on equal clusters) come from their own instantiation,
  // so the other calls' kernel carries none of their stores
  const size_t lds = (size_t)2 * t.d + sizeof(unsigned long long) * kRepairCap;
  if (mode == kTopkOnly)
    hipLaunchKernelGGL((topk_kernel<EPT, kSelIds>), dim3(G), dim3(kTopkThreads), 0, s, t);
  else if (approx && t.rank)
    hipLaunchKernelGGL((topk_kernel<EPT, kSelMark, true, true>), dim3(G), dim3(kTopkThreads), lds, s, t);
  else if (approx)
    hipLaunchKernelGGL((topk_kernel<EPT, kSelMark, false, true>), dim3(G), dim3(kTopkThreads), lds, s, t);
  else if (t.rank)
    hipLaunchKernelGGL((topk_kernel<EPT, kSelMark, true>), dim3(G), dim3(kTopkThreads), 0, s, t);
  else
    hipLaunchKernelGGL((topk_kernel<EPT, kSelMark>), dim3(G), dim3(kTopkThreads), 0, s, t);
}

hipError_t launch_topk(const PassArgs& a, int mode, hipStream_t s) {
  TopkArgs t;
  t.S = a.S;
  t.ldS = a.ldS;
  t.Nc = a.Nc;
  t.K = a.K;
  t.out = a.topk;
  t.ldK = a.ldK;
  t.cl_sel = a.cl_sel;
  t.best = a.best;
  t.amax = a.amax;
  t.rank = a.tm_rank;
  t.ldR = a.ldR;
  t.h = static_cast<const uint16_t*>(a.h);
  t.CT = static_cast<const v4u*>(a.t.CT);
  t.d = a.d;
  t.cmax = a.t.stats;
  t.stats = a.t.stats + kStatsCounters;
  t.hnorm = cert_gather(a) ? a.hnorm : nullptr;
  t.rows = a.B;
  t.fill = a.fill;
  t.fill_n = (long)a.B * a.V;
  const int G = a.B + fill_topk_groups(a);
  const bool approx = a.approx && mode != kTopkOnly;
  const int ept = (a.Nc + kTopkThreads - 1) / kTopkThreads;
  if (ept <= 1) launch_topk_ept<1>(t, G, mode, approx, s);
  else if (ept <= 2) launch_topk_ept<2>(t, G, mode, approx, s);
  else if (ept <= 4) launch_topk_ept<4>(t, G, mode, approx, s);
  else if (ept <= 8) launch_topk_ept<8>(t, G, mode, approx, s);
  else launch_topk_ept<16>(t, G, mode, approx, s);   // Nc <= kMaxNc: at most 16 keys a thread
  return hipGetLastError();
}

// Waves per tile (log2) for a pass of B rows.
// Below 48 rows a tile of the sweep head almost never needs a second pass
// (B=32: 33.3 µs per call split or not); at 64 rows the two-pass tiles set
// the gather's tail and splitting them takes the call from 39.2 to 37.8 µs.
static int gather_split_shift(int B) { return B >= 48 ? kGatherSplitShift : 0; }
// Ragged heads (the contiguous tiling): a tile shared by several clusters,
// or of a cluster many rows selected, needs several passes (skewed head,
// d=512, B=64: gather 44.3 µs with two waves a tile, 32.6 with four, 33.2
// with eight).
constexpr int kRaggedSplitShift = 2;
static int gather_split_shift_ragged(int B) { return B >= 16 ? kRaggedSplitShift : 0; }

// Largest batch whose float64 gather runs by row (equal clusters only):
// the B·K·tpc waves of the selected (row, centroid, tile) triples, every
// one with work, against the static grid of every tile, most of whose
// waves find no row.  A tile that several rows selected is then read once
// per row, which the batches below the split (48 rows) afford: sweep head,
// µs per call, B=8 19.8 → 16.6, B=16 22.0 → 19.0, B=32 27.3 → 24.1 (forward
// B=16 24.2 → 21.0, top-m B=16 26.7 → 23.0).  At B=64 the repeats cost more
// than the idle waves (33.2 → 36.7), except for FP8 slabs, whose argmax
// runs by row at every batch (B=64 27.8 → 26.0): with half the bytes a
// tile, the repeats cost less than the tile grid's uneven spread.  (On earlier kernels the limit measured best at
// 4 rows.)  Beyond 4 rows by row needs about one row per selected tile
// (B K <= 2 Nc, as on the sweep head, where it is 0.5 to 1): where rows
// share most tiles (K near Nc) every repeat is a slab read.
constexpr int kGatherByRowMaxB = 47;
constexpr int kGatherByRowAlways = 4;

template <typename T, int MODE>
static bool gather_by_row(const PassArgs& a) {
  if (a.t.tpc == 0) return false;
  if (a.B <= kGatherByRowAlways) return true;
  const bool fp8_argmax = std::is_same<T, uint8_t>::value && MODE == kArgmax;
  return (long)a.B * a.K <= 2l * a.Nc && (fp8_argmax || a.B <= kGatherByRowMaxB);
}
// Batches of at most this many rows on equal clusters keep the float64 dot
// by row even where the certified matrix-core argmax is on (a wave there
// holds a single row, which the float64 chain serves better); larger ones
// take the certified argmax's tile grid.
constexpr int kCertByRowMaxB = 4;

static bool cert_gather(const PassArgs& a) {
  return a.cert && !(a.t.tpc > 0 && a.B <= kCertByRowMaxB);
}

// Row groups of 16 per pass of the certified gather: where the selected
// tiles carry more than 16 rows on average (B K / Nc on equal clusters), a
// pass takes 32 or 64 rows, so each tile streams from memory once rather
// than once per 16 rows.
static int cert_row_groups(const PassArgs& a) {
  const long rows_per_tile = (long)a.B * a.K / a.Nc;
  if (a.t.tpc > 0 && rows_per_tile > 32) return 4;
  if (a.t.tpc > 0 && rows_per_tile > 16) return 2;
  return 1;
}

template <typename T, int MODE>
static hipError_t launch_gather_t(const PassArgs& a, hipStream_t s) {
  GatherArgs g;
  g.ET = static_cast<const v4u*>(a.t.ET);
  g.h = a.h;
  g.d = a.d;
  g.cl_sel = a.cl_sel;
  g.B = a.B;
  g.tcl = a.t.tcl;
  g.tpc = a.t.tpc;
  g.ttok = a.t.ttok;
  g.escale = a.t.escale;
  const bool by_row = gather_by_row<T, MODE>(a);
  g.split_shift = a.t.tpc > 0 ? (by_row ? 0 : gather_split_shift(a.B)) : gather_split_shift_ragged(a.B);
  g.best = a.best;
  g.amax = a.amax;
  g.out = a.logits;
  g.V = a.V;
  g.m = a.m;
  g.tm_keys = a.tm_keys;
  g.tm_heads = a.tm_heads;
  g.tm_cap = a.tm_cap;
  g.tm_segcap = a.tm_segcap;
  g.tm_rank = MODE == kTopM ? a.tm_rank : nullptr;
  g.ldR = a.ldR;
  g.n_tiles = a.t.n_tiles;
  g.topk = a.topk;
  g.ldK = a.ldK;
  g.K = a.K;
  g.by_row = by_row;
  g.enorm = a.t.enorm;
  g.crec = reinterpret_cast<v4u*>(a.crec);
  g.crank = a.tm_rank;
  g.hnorm = a.hnorm;
  if constexpr (MODE == kArgmax && !std::is_same<T, float>::value) {
    if (cert_gather(a)) {
      // a pass holds 16 rows; where a tile carries more on average (B K / Nc
      // of them), its passes go to 2 or 4 waves, which share the XCD's L2
      // (slot-major grid, n_tiles a multiple of 8 on large heads).  Ragged
      // heads' correlated rows pile onto a few tiles: from 17 rows their
      // passes take two waves (skewed head, B=64: gather 24.0 -> 17.2 µs,
      // call 40.3 -> 32.9; four waves the same)
      const long rows_per_tile = (long)a.B * a.K / a.Nc;
      const int rg = cert_row_groups(a);
      g.split_shift = rg > 1 ? 0
                      : (rows_per_tile > 16 || (a.t.tpc == 0 && a.B > 16)) ? 1
                                                                         : 0;
      const dim3 cgrid((unsigned)a.t.n_tiles << g.split_shift);
      auto go_cert = [&](auto kern) {
        if (a.probe_start && a.probe_stop)
          hipExtLaunchKernelGGL(kern, cgrid, dim3(64), 0, s, a.probe_start, a.probe_stop, 0, g);
        else
          hipLaunchKernelGGL(kern, cgrid, dim3(64), 0, s, g);
      };
#define CE_CERT(RGN)                                                  \
  switch (a.d / 32) {                                                 \
    case 8: go_cert(gather_cert_kernel<T, 8, RGN>); break;            \
    case 16: go_cert(gather_cert_kernel<T, 16, RGN>); break;          \
    case 32: go_cert(gather_cert_kernel<T, 32, RGN>); break;          \
    default: go_cert(gather_cert_kernel<T, 0, RGN>); break;           \
  }
      if (rg == 4 && a.d <= kCertHlMaxD) {
        // the persistent kernel with the pass's rows in LDS
        const unsigned groups = (unsigned)std::min<long>(
            kCertHlGroups, ((long)a.t.n_tiles + kCertHlWaves - 1) / kCertHlWaves);
        const size_t lds = (size_t)a.B * (2 * a.d + 16);
        auto go_hl = [&](auto kern) {
          (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
          if (a.probe_start && a.probe_stop)
            hipExtLaunchKernelGGL(kern, dim3(groups), dim3(64 * kCertHlWaves), lds, s, a.probe_start,
                                  a.probe_stop, 0, g);
          else
            hipLaunchKernelGGL(kern, dim3(groups), dim3(64 * kCertHlWaves), lds, s, g);
        };
        // (d = 1024 takes the rolled pipeline: unrolled, its 32 blocks
        // would not fit the registers)
        switch (a.d / 32) {
          case 8: go_hl(gather_cert_hl_kernel<T, 8>); break;
          case 16: go_hl(gather_cert_hl_kernel<T, 16>); break;
          default: go_hl(gather_cert_hl_kernel<T, 0>); break;
        }
      } else if (rg == 4) CE_CERT(4)
      else if (rg == 2) CE_CERT(2)
      else CE_CERT(1)
#undef CE_CERT
      return hipGetLastError();
    }
  }
  const dim3 grid(g.by_row ? (unsigned)(a.B * a.K * a.t.tpc)
                           : a.t.n_tiles > 0 ? (unsigned)a.t.n_tiles << g.split_shift : 1u);
  auto go = [&](auto kern) {
    if (a.probe_start && a.probe_stop) {
      hipExtLaunchKernelGGL(kern, grid, dim3(64), 0, s, a.probe_start, a.probe_stop, 0, g);
    } else {
      hipLaunchKernelGGL(kern, grid, dim3(64), 0, s, g);
    }
  };
  // by row a wave dots a single row: the one-row instantiation skips the
  // three unused row slots' hidden loads, widening and branches (B=1..4:
  // 0.4–0.9 µs per call on every entry point)
#define CE_GATHER(N)                                                                           \
  (g.by_row            ? go(gather_kernel<T, 1, MODE, N, kGatherStagesByRow<T>>)                   \
   : g.split_shift > 0 ? go(gather_kernel<T, kGatherRows, MODE, N, kGatherStages<T, MODE, true>>)  \
                       : go(gather_kernel<T, kGatherRows, MODE, N, kGatherStages<T, MODE, false>>))
  CE_DISPATCH_NCH(a.d, CE_GATHER)
#undef CE_GATHER
  return hipGetLastError();
}

hipError_t launch_gather(const PassArgs& a, int mode, hipStream_t s) {
  if (a.t.n_tiles == 0) return hipSuccess;   // every cluster is empty
  if (a.t.slab == 1) {
    if (mode == kArgmax) return launch_gather_t<uint8_t, kArgmax>(a, s);
    if (mode == kMasked) return launch_gather_t<uint8_t, kMasked>(a, s);
    return launch_gather_t<uint8_t, kTopM>(a, s);
  }
  if (a.dtype == 1) {
    if (mode == kArgmax) return launch_gather_t<uint16_t, kArgmax>(a, s);
    if (mode == kMasked) return launch_gather_t<uint16_t, kMasked>(a, s);
    return launch_gather_t<uint16_t, kTopM>(a, s);
  }
  if (mode == kArgmax) return launch_gather_t<float, kArgmax>(a, s);
  if (mode == kMasked) return launch_gather_t<float, kMasked>(a, s);
  return launch_gather_t<float, kTopM>(a, s);
}

hipError_t launch_topm_merge(const PassArgs& a, hipStream_t s) {
  TopmArgs t;
  t.cnt = a.best;
  t.keys = a.tm_keys;
  t.heads = a.tm_heads;
  t.cap = a.tm_cap;
  t.segcap = a.tm_segcap;
  t.m = a.m;
  t.fixed_segs = a.tm_rank ? a.K * a.t.tpc : 0;
  t.tokens = a.tm_tokens;
  t.logits = a.tm_logits;
  t.log_softmax = a.tm_log_softmax ? 1 : 0;
  const size_t lds = ((size_t)a.tm_segcap + (size_t)a.m * kTileTokens) * sizeof(unsigned long long);
  hipLaunchKernelGGL(topm_merge_kernel, dim3(a.B), dim3(kTopkThreads), lds, s, t);
  return hipGetLastError();
}

// Streaming-read probe: every 16-byte vector of the buffer is loaded once,
// eight independent non-temporal loads per thread per step, grid-stride; the
// XOR of the loaded words feeds a store that never happens for real data
// (sink is written only if it equals an improbable pattern), so no load is
// dropped.  Of the configurations measured on a 2 GiB buffer (two to sixteen
// loads in flight, 4096 to 32768 workgroups of 256 threads, plain and
// non-temporal loads) this one read fastest: 6.37 TB/s, against 5.9 TB/s at
// best with plain loads.
constexpr int kProbeLoads = 8;
__global__ __launch_bounds__(256) void stream_read_kernel(const v4u* __restrict__ p, long n,
                                                          uint32_t* __restrict__ sink) {
  const long stride = (long)gridDim.x * blockDim.x;
  long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeLoads - 1) * stride < n; i += kProbeLoads * stride) {
    v4u v[kProbeLoads];
#pragma unroll
    for (int u = 0; u < kProbeLoads; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeLoads; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const v4u a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  const long n = (long)(bytes / sizeof(v4u));
  if (n == 0) return hipSuccess;
  // 32 workgroups of 256 threads per CU on the 256-CU part; fewer when the
  // buffer is small, so every thread has at least one vector
  const long blocks = std::min<long>(8192, (n + 255) / 256);
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const v4u*>(buf), n, sink);
  return hipGetLastError();
}

hipError_t launch_finalize(const PassArgs& a, hipStream_t s) {
  if (a.emb_table) {
    EmbedArgs e{a.emb_table, a.emb_dim, a.emb_normalizer, a.emb_out};
    if (a.dtype == 1)
      hipLaunchKernelGGL(finalize_embed_kernel<uint16_t>, dim3(a.B), dim3(kEmbedThreads), 0, s,
                         a.amax, a.tokens, e);
    else
      hipLaunchKernelGGL(finalize_embed_kernel<float>, dim3(a.B), dim3(kEmbedThreads), 0, s,
                         a.amax, a.tokens, e);
  } else if (cert_gather(a)) {
    CertArgs f{reinterpret_cast<const v4u*>(a.crec), a.t.n_tiles, static_cast<const v4u*>(a.t.ET),
               a.t.escale, a.t.ttok, a.t.tcl, a.cl_sel, static_cast<const uint16_t*>(a.h), a.d,
               a.topk, a.ldK, a.K, a.t.offsets, a.t.tpc, a.tokens};
    const size_t lds = (size_t)2 * a.d;
    if (a.t.slab == 1)
      hipLaunchKernelGGL(finalize_cert_kernel<uint8_t>, dim3(a.B), dim3(kCertThreads), lds, s, f);
    else
      hipLaunchKernelGGL(finalize_cert_kernel<uint16_t>, dim3(a.B), dim3(kCertThreads), lds, s, f);
  } else {
    hipLaunchKernelGGL(finalize_kernel, dim3((a.B + 63) / 64), dim3(64), 0, s, a.amax, a.B, a.tokens);
  }
  return hipGetLastError();
}

hipError_t launch_slot_norms(const void* ET, int slab, const float* escale, long n_tiles, int d,
                             float* out, hipStream_t s) {
  const long n = n_tiles * kWave;
  if (n == 0) return hipSuccess;
  long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (slab == 1)
    hipLaunchKernelGGL(slot_norm_kernel<uint8_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const v4u*>(ET), escale, n, d, out);
  else
    hipLaunchKernelGGL(slot_norm_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const v4u*>(ET), escale, n, d, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ static scratch

// The workspace of ce_top_tokens_static, for callers that cannot allocate:
// one array per GPU, held by the library until the process ends.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the array's name is a host-side stand-in: its device address on the
    // current device comes from the runtime, once per device
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace ce
