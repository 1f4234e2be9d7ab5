// HIP kernels of the centroid-masked sparse LM head, written for CDNA4 (gfx950).
//
// The operation is Gemma4MTPMaskedEmbedder of the vLLM compare view "[Spec
// Decode] Add Gemma4 MTP speculative decoding with centroids masking" (diff of
// gemma4_mtp.py): centroid projection, top-K centroids, gather of the tokens
// the selected centroids own (ordered-embedding layout), sparse dot products,
// then a greedy argmax (get_top_tokens) or a full-vocabulary row filled with
// -inf outside the candidates (forward).
//
// One pass handles at most 64 rows and runs these kernels in stream order:
//   prep     widen h to float64, clear the per-call counters and row masks
//   scores   centroid projection S[b][c] (canonical dot, see below)
//   topk     one workgroup per row: radix select of the K best centroids; the
//            first row to claim a centroid appends its 64-token tiles to the
//            gather work list (cross-row dedup: each tile is read once)
//   gather   one wave per 64-token tile: stage the tile through LDS once, dot
//            every row that selected its centroid, then either reduce to a
//            per-row packed argmax with a 64-bit atomicMax (the last tile to
//            finish writes the token ids) or store the candidate logits
//   writer   (forward only) one coalesced pass over [B][V]: -inf or the
//            candidate logit of each token
//
// Canonical dot: every product is formed exactly in float64 and summed in
// hidden-dimension order from +0.0 by a chain of v_fmac_f64 (one rounding per
// step), then rounded to fp32 nearest-even with -0 mapped to +0.  Each lane
// owns whole chains (one per output), so no reduction tree reorders a sum and
// the results equal a sequential float64 loop bit for bit.  The hidden rows are
// wave-uniform operands: they are read as float64 through the scalar cache
// (address space 4) and fed to v_fmac_f64 as SGPR pairs.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "ce_internal.h"

namespace ce {
namespace {

constexpr int kWave = 64;
constexpr int kChunk = 64;   // hidden dims staged through LDS per step

typedef const __attribute__((address_space(4))) double cdouble_t;

// 16 bytes as a native vector (HIP's uint4 wraps a union, which keeps arrays
// of it out of registers).
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// View of read-only float64 data as the constant address space, so that
// wave-uniform reads become scalar loads.
__device__ __forceinline__ cdouble_t* as_const(const double* p) { return (cdouble_t*)p; }

template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int kPerVec = 4; };      // fp32
template <> struct Elem<uint16_t> { static constexpr int kPerVec = 8; };   // bf16 bits

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

__device__ __forceinline__ double widen1(float v) { return (double)v; }
__device__ __forceinline__ double widen1(uint16_t v) {
  return (double)__uint_as_float((uint32_t)v << 16);
}

// float64 sum -> fp32 nearest-even, -0 -> +0.
__device__ __forceinline__ float canon(double s) {
  uint32_t u = __float_as_uint((float)s);
  return __uint_as_float(u == 0x80000000u ? 0u : u);
}

// Order-preserving map of a (non-NaN) fp32 to u32; -0 and +0 map alike.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T>
struct TileGeom {
  static constexpr int kPerVec = Elem<T>::kPerVec;
  static constexpr int kVecPerTok = kChunk / kPerVec;      // 16-byte vectors per token per chunk
  static constexpr int kTokStep = kWave / kVecPerTok;      // tokens covered by one wave load
  static constexpr int kLoads = kVecPerTok;                // loads per lane per chunk
  static constexpr int kPitch = kVecPerTok + 1;            // LDS row pitch in 16-byte units (+16 B pad)
  static constexpr int kLdsVecs = kTileTokens * kPitch;
};

// Dot 64 consecutive rows of W ([*, d] row-major) starting at row j0 (rows
// >= nvalid are clamped to nvalid-1 and their results must be ignored) with
// up to RB hidden rows hrow[0..nrows) (float64, scalar-cache reads).  Lane t
// ends with acc[r] = the float64 chain for (row j0+t, hidden row r).
//
// Each chunk of 64 dims is read from HBM with fully coalesced 16-byte loads
// (8 tokens x 128 B per wave instruction for bf16), written to LDS with a
// 16-byte pad per token row so that the per-lane row reads are bank-conflict
// free, and the next chunk's loads are in flight while this one is consumed.
template <typename T, int RB>
__device__ __forceinline__ void dot_tile(const T* __restrict__ W, long j0, int nvalid, int d,
                                         cdouble_t* const (&hrow)[RB], int nrows,
                                         double (&acc)[RB], v4u* lds) {
  using G = TileGeom<T>;
  const int lane = threadIdx.x;
  const int part = lane % G::kVecPerTok;
  const int tok0 = lane / G::kVecPerTok;
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = 0.0;

  const v4u* src[G::kLoads];
#pragma unroll
  for (int i = 0; i < G::kLoads; ++i) {
    int tok = tok0 + i * G::kTokStep;
    tok = tok < nvalid ? tok : nvalid - 1;
    src[i] = reinterpret_cast<const v4u*>(W + (j0 + tok) * (long)d) + part;
  }
  v4u buf[G::kLoads];
#pragma unroll
  for (int i = 0; i < G::kLoads; ++i) buf[i] = src[i][0];

  // consume the chunk staged in LDS: dims [kc, kc + kChunk)
  auto consume = [&](int kc) {
#pragma unroll
    for (int p = 0; p < G::kVecPerTok; ++p) {
      const v4u v = lds[lane * G::kPitch + p];
      double x[G::kPerVec];
      widen(v, x, T());
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (r < nrows) {
          cdouble_t* hp = hrow[r] + kc + p * G::kPerVec;
#pragma unroll
          for (int i = 0; i < G::kPerVec; ++i) acc[r] = __builtin_fma(x[i], hp[i], acc[r]);
        }
      }
    }
  };

  const int last = d / kChunk - 1;
  for (int ch = 0; ch < last; ++ch) {
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) lds[(tok0 + i * G::kTokStep) * G::kPitch + part] = buf[i];
    __syncthreads();
    const int adv = (ch + 1) * (kChunk / G::kPerVec);
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) buf[i] = src[i][adv];   // next chunk in flight
    consume(ch * kChunk);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < G::kLoads; ++i) lds[(tok0 + i * G::kTokStep) * G::kPitch + part] = buf[i];
  __syncthreads();
  consume(last * kChunk);
  __syncthreads();
}

// ------------------------------------------------------------------ prep

template <typename T>
__global__ __launch_bounds__(256) void prep_kernel(const T* __restrict__ h, int n, double* H64,
                                                   int Nc, unsigned long long* cl_mask,
                                                   unsigned long long* best, CallState* st) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int stride = gridDim.x * blockDim.x;
  for (int k = i; k < n; k += stride) H64[k] = widen1(h[k]);
  if (cl_mask)
    for (int k = i; k < Nc; k += stride) cl_mask[k] = 0ull;
  if (i < kPassRows) {
    if (best) best[i] = 0ull;
    reinterpret_cast<uint32_t*>(st)[i] = 0u;
  }
}

// ------------------------------------------------------------------ scores

template <typename T, int RB>
__global__ __launch_bounds__(64) void scores_kernel(const T* __restrict__ C, int Nc, int d,
                                                    const double* __restrict__ H64, int B,
                                                    float* __restrict__ S, int ldS) {
  __shared__ v4u lds[TileGeom<T>::kLdsVecs];
  const int c0 = blockIdx.x * kTileTokens;
  const int r0 = blockIdx.y * RB;
  const int nvalid = min(kTileTokens, Nc - c0);
  const int nrows = min(RB, B - r0);
  cdouble_t* hrow[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
    hrow[r] = as_const(H64 + (long)(r0 + (r < nrows ? r : nrows - 1)) * d);
  double acc[RB];
  dot_tile<T, RB>(C, c0, nvalid, d, hrow, nrows, acc, lds);
  const int lane = threadIdx.x;
  if (lane < nvalid) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
      if (r < nrows) S[(long)(r0 + r) * ldS + c0 + lane] = canon(acc[r]);
  }
}

// ------------------------------------------------------------------ top-K

constexpr int kTopkThreads = 256;

// Exclusive prefix sum over the 256 threads of the block; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) sh[w] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kTopkThreads / kWave; ++i) {
    const uint32_t s = sh[i];
    base += (i < w) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

struct TopkArgs {
  const float* S;
  int ldS, Nc, K;
  int32_t* out;
  int ldK;
  int b_base;                      // row index offset into cl_mask bit positions (0)
  const int32_t* offsets;
  unsigned long long* cl_mask;
  uint32_t* items;
  CallState* st;
  int32_t* rowpos;
};

// One workgroup per row.  Thread t holds centroids [t*EPT, t*EPT+EPT), so
// thread order is id order.  MSB-first radix select over 8-bit digits finds
// the exact K-th largest key tau and how many keys equal to tau to keep; the
// kept ties are the lowest ids.  The result is written in ascending id order.
template <int EPT, int MODE>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  static_assert(EPT <= 32, "selection mask is 32 bits");
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_sh[kTopkThreads / kWave];
  __shared__ uint32_t sel_digit, sel_kk;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int Nc = a.Nc;
  const float* row = a.S + (long)b * a.ldS;

  uint32_t key[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int c = tid * EPT + i;
    key[i] = c < Nc ? order_key(row[c]) : 0u;
  }

  uint32_t prefix = 0, pmask = 0, kk = (uint32_t)a.K;
  const bool take_all = a.K >= Nc;
  if (!take_all) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const int c = tid * EPT + i;
        if (c < Nc && (key[i] & pmask) == prefix) atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
      }
      __syncthreads();
      // thread t looks at digit 255-t: excl = keys with a larger digit
      const uint32_t v = hist[255 - tid];
      uint32_t tot;
      const uint32_t excl = block_excl_scan(v, scan_sh, &tot);
      if (excl < kk && excl + v >= kk) {
        sel_digit = 255u - (uint32_t)tid;
        sel_kk = kk - excl;
      }
      __syncthreads();
      prefix |= sel_digit << shift;
      pmask |= 0xFFu << shift;
      kk = sel_kk;
    }
  }
  const uint32_t tau = prefix;

  // tie ranks in id order
  uint32_t n_eq = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int c = tid * EPT + i;
    n_eq += (c < Nc && key[i] == tau) ? 1u : 0u;
  }
  uint32_t tot;
  uint32_t eq_seen = block_excl_scan(n_eq, scan_sh, &tot);
  uint32_t selmask = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int c = tid * EPT + i;
    bool s = false;
    if (c < Nc) {
      if (take_all || key[i] > tau) {
        s = true;
      } else if (key[i] == tau) {
        s = eq_seen < kk;
        ++eq_seen;
      }
    }
    selmask |= (s ? 1u : 0u) << i;
  }
  uint32_t pos = block_excl_scan((uint32_t)__popc(selmask), scan_sh, &tot);
  int32_t* out = a.out + (long)b * a.ldK;
#pragma unroll
  for (int i = 0; i < EPT; ++i)
    if (selmask & (1u << i)) out[pos++] = tid * EPT + i;

  if (MODE >= kTopkPlan) {
    const unsigned long long bit = 1ull << b;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      if (selmask & (1u << i)) {
        const int c = tid * EPT + i;
        const unsigned long long old = atomicOr(&a.cl_mask[c], bit);
        if (old == 0ull) {
          const int n = a.offsets[c + 1] - a.offsets[c];
          const uint32_t nt = (uint32_t)((n + kTileTokens - 1) / kTileTokens);
          if (nt) {
            const uint32_t base = atomicAdd(&a.st->n_items, nt);
            for (uint32_t q = 0; q < nt; ++q)
              a.items[base + q] = (q << kItemShift) | (uint32_t)c;
          }
        }
      }
    }
  }
  if (MODE == kTopkPlanRowpos) {
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i)
      if (selmask & (1u << i)) {
        const int c = tid * EPT + i;
        local += (uint32_t)(a.offsets[c + 1] - a.offsets[c]);
      }
    uint32_t run = block_excl_scan(local, scan_sh, &tot);
    int32_t* rp = a.rowpos + (long)b * Nc;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int c = tid * EPT + i;
      if (c < Nc) {
        if (selmask & (1u << i)) {
          rp[c] = (int32_t)run;
          run += (uint32_t)(a.offsets[c + 1] - a.offsets[c]);
        } else {
          rp[c] = -1;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ gather

struct GatherArgs {
  const void* E;
  int d, Nc, B;
  const int32_t* offsets;
  const int32_t* tos;
  const double* H64;
  const unsigned long long* cl_mask;
  const uint32_t* items;
  CallState* st;
  unsigned long long* best;
  int32_t* tokens;
  const int32_t* rowpos;
  float* L;
  int ldL;
};

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const unsigned long long w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

template <typename T, int RB, int MODE>
__global__ __launch_bounds__(64) void gather_kernel(GatherArgs a) {
  __shared__ v4u lds[TileGeom<T>::kLdsVecs];
  const int lane = threadIdx.x;
  const uint32_t n_items = a.st->n_items;
  const uint32_t it = blockIdx.x;
  if (it >= n_items) {
    if (MODE == kArgmax && it == 0) {
      // no work at all: every row's selected centroids are empty
      for (int b = lane; b < a.B; b += kWave) a.tokens[b] = -1;
    }
    return;
  }
  const uint32_t item = a.items[it];
  const int c = (int)(item & ((1u << kItemShift) - 1u));
  const int q = (int)(item >> kItemShift);
  const long j0 = (long)a.offsets[c] + (long)q * kTileTokens;
  const int nvalid = (int)min((long)kTileTokens, (long)a.offsets[c + 1] - j0);
  const int tok = lane < nvalid ? a.tos[j0 + lane] : 0;
  unsigned long long mask = a.cl_mask[c];
  const T* E = reinterpret_cast<const T*>(a.E);

  while (mask) {
    int rows[RB];
    int nrows = 0;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (mask) {
        rows[r] = __builtin_ctzll(mask);
        mask &= mask - 1ull;
        ++nrows;
      } else {
        rows[r] = rows[0];
      }
    }
    cdouble_t* hrow[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) hrow[r] = as_const(a.H64 + (long)rows[r] * a.d);
    double acc[RB];
    dot_tile<T, RB>(E, j0, nvalid, a.d, hrow, nrows, acc, lds);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (r < nrows) {
        const float f = canon(acc[r]);
        if (MODE == kArgmax) {
          unsigned long long k = 0ull;
          if (lane < nvalid)
            k = ((unsigned long long)order_key(f) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)tok);
          k = wave_max_u64(k);
          if (lane == 0) atomicMax(&a.best[rows[r]], k);
        } else {
          if (lane < nvalid) {
            const int p = a.rowpos[(long)rows[r] * a.Nc + c];
            a.L[(long)rows[r] * a.ldL + p + q * kTileTokens + lane] = f;
          }
        }
      }
    }
  }

  if (MODE == kArgmax) {
    // completion ticket: the last item to finish decodes every row's winner
    __threadfence();
    uint32_t ticket = 0;
    if (lane == 0) ticket = atomicAdd(&a.st->done_items, 1u);
    ticket = __shfl(ticket, 0, kWave);
    if (ticket == n_items - 1u) {
      __threadfence();
      for (int b = lane; b < a.B; b += kWave) {
        const unsigned long long v =
            __hip_atomic_load(&a.best[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        a.tokens[b] = v ? (int32_t)(0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFull)) : -1;
      }
    }
  }
}

// ------------------------------------------------------------------ writer

constexpr int kWriterRows = 8;

// out[b][t] for 4 consecutive tokens t and kWriterRows rows per thread:
// the candidate logit when t's centroid is selected by row b, else -inf.
__global__ __launch_bounds__(256) void writer_kernel(float* __restrict__ out, int B, int V, int Nc,
                                                     const int32_t* __restrict__ tok_cluster,
                                                     const int32_t* __restrict__ tok_rank,
                                                     const int32_t* __restrict__ rowpos,
                                                     const float* __restrict__ L, int ldL) {
  const long t0 = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (t0 >= V) return;
  const int n = (int)min(4L, (long)V - t0);
  int cl[4], rk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cl[i] = i < n ? tok_cluster[t0 + i] : 0;
    rk[i] = i < n ? tok_rank[t0 + i] : 0;
  }
  const int b0 = blockIdx.y * kWriterRows;
  const bool vec = (n == 4) && ((V & 3) == 0);
#pragma unroll
  for (int rr = 0; rr < kWriterRows; ++rr) {
    const int b = b0 + rr;
    if (b < B) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = -__builtin_inff();
        if (i < n) {
          const int p = rowpos[(long)b * Nc + cl[i]];
          if (p >= 0) v[i] = L[(long)b * ldL + p + rk[i]];
        }
      }
      float* o = out + (long)b * V + t0;
      if (vec) {
        *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        for (int i = 0; i < n; ++i) o[i] = v[i];
      }
    }
  }
}

}  // namespace

// ------------------------------------------------------------------ launchers

hipError_t launch_prep(const PassArgs& a, hipStream_t s) {
  const int n = a.B * a.d;
  const int work = n > a.Nc ? n : a.Nc;
  int blocks = (work + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  if (a.dtype == 1)
    hipLaunchKernelGGL(prep_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(a.h), n, a.H64, a.Nc, a.cl_mask, a.best, a.state);
  else
    hipLaunchKernelGGL(prep_kernel<float>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const float*>(a.h), n, a.H64, a.Nc, a.cl_mask, a.best, a.state);
  return hipGetLastError();
}

template <typename T, int RB>
static void launch_scores_t(const PassArgs& a, hipStream_t s) {
  const dim3 grid((a.Nc + kTileTokens - 1) / kTileTokens, (a.B + RB - 1) / RB);
  hipLaunchKernelGGL((scores_kernel<T, RB>), grid, dim3(64), 0, s, static_cast<const T*>(a.C),
                     a.Nc, a.d, a.H64, a.B, a.S, a.ldS);
}

hipError_t launch_scores(const PassArgs& a, hipStream_t s) {
  // two rows per wave once there are enough rows to keep the chip busy
  const bool two = a.B >= 2;
  if (a.dtype == 1) {
    if (two) launch_scores_t<uint16_t, 2>(a, s); else launch_scores_t<uint16_t, 1>(a, s);
  } else {
    if (two) launch_scores_t<float, 2>(a, s); else launch_scores_t<float, 1>(a, s);
  }
  return hipGetLastError();
}

template <int EPT>
static void launch_topk_ept(const TopkArgs& t, int B, int mode, hipStream_t s) {
  if (mode == kTopkOnly)
    hipLaunchKernelGGL((topk_kernel<EPT, kTopkOnly>), dim3(B), dim3(kTopkThreads), 0, s, t);
  else if (mode == kTopkPlan)
    hipLaunchKernelGGL((topk_kernel<EPT, kTopkPlan>), dim3(B), dim3(kTopkThreads), 0, s, t);
  else
    hipLaunchKernelGGL((topk_kernel<EPT, kTopkPlanRowpos>), dim3(B), dim3(kTopkThreads), 0, s, t);
}

hipError_t launch_topk(const PassArgs& a, int mode, hipStream_t s) {
  TopkArgs t;
  t.S = a.S;
  t.ldS = a.ldS;
  t.Nc = a.Nc;
  t.K = a.K;
  t.out = a.topk;
  t.ldK = a.ldK;
  t.b_base = 0;
  t.offsets = a.t.offsets;
  t.cl_mask = a.cl_mask;
  t.items = a.items;
  t.st = a.state;
  t.rowpos = a.rowpos;
  const int ept = (a.Nc + kTopkThreads - 1) / kTopkThreads;
  if (ept <= 1) launch_topk_ept<1>(t, a.B, mode, s);
  else if (ept <= 2) launch_topk_ept<2>(t, a.B, mode, s);
  else if (ept <= 4) launch_topk_ept<4>(t, a.B, mode, s);
  else if (ept <= 8) launch_topk_ept<8>(t, a.B, mode, s);
  else if (ept <= 16) launch_topk_ept<16>(t, a.B, mode, s);
  else launch_topk_ept<32>(t, a.B, mode, s);
  return hipGetLastError();
}

template <typename T, int MODE>
static hipError_t launch_gather_t(const PassArgs& a, hipStream_t s) {
  GatherArgs g;
  g.E = a.E;
  g.d = a.d;
  g.Nc = a.Nc;
  g.B = a.B;
  g.offsets = a.t.offsets;
  g.tos = a.t.tos;
  g.H64 = a.H64;
  g.cl_mask = a.cl_mask;
  g.items = a.items;
  g.st = a.state;
  g.best = a.best;
  g.tokens = a.tokens;
  g.rowpos = a.rowpos;
  g.L = a.L;
  g.ldL = a.ldL;
  const dim3 grid(a.max_items > 0 ? a.max_items : 1);
  auto kern = gather_kernel<T, 8, MODE>;
  if (a.probe_start && a.probe_stop) {
    hipExtLaunchKernelGGL(kern, grid, dim3(64), 0, s, a.probe_start, a.probe_stop, 0, g);
  } else {
    hipLaunchKernelGGL(kern, grid, dim3(64), 0, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const PassArgs& a, int mode, hipStream_t s) {
  if (a.dtype == 1)
    return mode == kArgmax ? launch_gather_t<uint16_t, kArgmax>(a, s)
                           : launch_gather_t<uint16_t, kMasked>(a, s);
  return mode == kArgmax ? launch_gather_t<float, kArgmax>(a, s)
                         : launch_gather_t<float, kMasked>(a, s);
}

hipError_t launch_writer(const PassArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.V + 1023) / 1024), (unsigned)((a.B + kWriterRows - 1) / kWriterRows));
  hipLaunchKernelGGL(writer_kernel, grid, dim3(256), 0, s, a.logits, a.B, a.V, a.Nc,
                     a.t.tok_cluster, a.t.tok_rank, a.rowpos, a.L, a.ldL);
  return hipGetLastError();
}

}  // namespace ce
