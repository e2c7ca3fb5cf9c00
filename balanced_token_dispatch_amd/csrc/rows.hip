// Row-streaming kernels: gather-permute, weighted combine, replica-gradient
// fold and slot prefetch.  All are HBM-bound and move whole rows with 16-byte
// vector loads/stores.  Every kernel is launched one-shot: a block owns one
// row (or one 16 KB chunk of a long row) and exits, so the hardware
// dispatcher keeps every CU saturated with fresh loads; a persistent
// grid-stride loop over rows measured 10-15 points of HBM peak slower on
// gfx950.  Both grid axes are clamped and the kernels stride past the clamp,
// so any row count or width is covered.  Loads and stores of rows are
// non-temporal (measured on the layer step's buffers: the permute's token-row
// reads 3% faster so, the router-weight gradient's output-gradient reads 16%,
// the combine's gathers 29% faster than plain loads), except the fold's
// read-modify-write of the home rows (4% slower non-temporal) and the gated
// unit's backward.
//
// Pages: moses-y.github.io "MoonEP", "What This Does" and "Real-World Use";
// findrepo.work "MoonEP" card, "Strengths" (fused permute / unpermute);
// ainovat.com "Moonshot AI Open-Sources MoonEP", mechanism paragraph
// (replica weights fetched ahead, replica gradients returned home).
#include "common.hpp"

namespace moe {

constexpr int kRowThreads = 256;      // combine / fold / prefetch blocks
constexpr int kPermMaxThreads = 1024; // permute: one block spans a whole row
// Combine / un-permute reduce blocks: kCombU vectors per thread, the block sized to the row
// (whole wavefronts, at most kCombMaxThreads), so a 14 KB bf16 row of 896 vectors is 448
// threads with no idle lane; 4 vectors on 256 threads (the last pass half idle) measured
// 3-4% slower, one vector per thread on 896 threads 8% slower.
constexpr int kCombU = 2;
constexpr int kCombMaxThreads = 1024;
inline int comb_threads(int vec) {
  const int t = (vec + kCombU - 1) / kCombU;
  return t >= kCombMaxThreads ? kCombMaxThreads : (t + 63) / 64 * 64;
}
constexpr int kStreamU = 4;           // vectors per thread per fold / prefetch block
constexpr int kMaxGridX = 1 << 20;
constexpr int kMaxGridY = 65535;

__device__ inline u32x4 scale_row16(u32x4 v, float w, bool bf16) {
  if (bf16) {
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = pack_bf16x2(w * bf16_lo(v[q]), w * bf16_hi(v[q]));
    return r;
  }
  f32x4 f = __builtin_bit_cast(f32x4, v);
  f *= w;
  return __builtin_bit_cast(u32x4, f);
}

// xp[i] = x_all[src_flat[i] / K] (optionally * row_scale[src]).  grid (row groups, chunks),
// block = kPermRows rows x one chunk of up to kPermMaxThreads vectors, one vector of each row
// per thread.
template <bool SCALED>
constexpr int kPermRows = SCALED ? 2 : 1;

template <bool SCALED>
__global__ __launch_bounds__(kPermMaxThreads) void k_permute(const u32x4 *__restrict__ x_all,
                                                            const int32_t *__restrict__ src_flat,
                                                            const float *__restrict__ scale,
                                                            u32x4 *__restrict__ xp, int SK, int K,
                                                            int vec_per_row, int bf16) {
  // the weighted form takes two rows per block: both rows' loads are in flight before the
  // multiplies (measured 8% faster; the plain copy gains nothing from it)
  constexpr int ROWS = kPermRows<SCALED>;
  for (int i0 = blockIdx.x * ROWS; i0 < SK; i0 += gridDim.x * ROWS) {
    int src[ROWS];
    float w[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      src[r] = i0 + r < SK ? src_flat[i0 + r] : -1;
      w[r] = (SCALED && src[r] >= 0) ? scale[src[r]] : 1.0f;
    }
    for (int v = blockIdx.y * blockDim.x + threadIdx.x; v < vec_per_row;
         v += gridDim.y * blockDim.x) {
      u32x4 t[ROWS];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        t[r] = (u32x4){0, 0, 0, 0};
        if (src[r] >= 0)
          t[r] = __builtin_nontemporal_load(x_all + (size_t)(src[r] / K) * vec_per_row + v);
      }
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        if (SCALED) t[r] = scale_row16(t[r], w[r], bf16);
        if (i0 + r < SK) __builtin_nontemporal_store(t[r], xp + (size_t)(i0 + r) * vec_per_row + v);
      }
    }
  }
}

constexpr int kMaxKUnrolled = 16;

template <bool BF16>
__device__ inline void fma_row16(float (&acc)[8], float w, u32x4 t) {
  if (BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = __builtin_fmaf(w, bf16_lo(t[q]), acc[2 * q]);
      acc[2 * q + 1] = __builtin_fmaf(w, bf16_hi(t[q]), acc[2 * q + 1]);
    }
  } else {
    const f32x4 f = __builtin_bit_cast(f32x4, t);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(w, f[q], acc[q]);
  }
}

template <bool BF16>
__device__ inline u32x4 round_row16(const float (&acc)[8]) {
  u32x4 r;
  if (BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
  } else {
    r = __builtin_bit_cast(u32x4, (f32x4){acc[0], acc[1], acc[2], acc[3]});
  }
  return r;
}

// out[s] = sum_k w[c] * y_all[dest_pos[c]], c = (rank*S + s)*K + k.  grid (tokens, chunks);
// a block covers blockDim.x*kCombU vectors of one token, all K source rows in flight.
// Without WEIGHTED every weight is 1 (the un-permute reduce of the dispatch's backward): the
// fused multiply-add by 1 rounds exactly like a plain add.
template <bool BF16, bool WEIGHTED = true>
__global__ __launch_bounds__(kCombMaxThreads) void k_combine(const u32x4 *__restrict__ y_all,
                                                        const int32_t *__restrict__ dest_pos,
                                                        const float *__restrict__ topk_w,
                                                        u32x4 *__restrict__ out, int S, int K,
                                                        int rank, int vec_per_row) {
  const int T = blockDim.x, kChunk = T * kCombU;
  for (int s = blockIdx.x; s < S; s += gridDim.x) {
    const size_t c0 = ((size_t)rank * S + s) * K;
    int dst[kMaxKUnrolled];
    float wt[kMaxKUnrolled];
#pragma unroll
    for (int k = 0; k < kMaxKUnrolled; ++k) {
      dst[k] = (k < K) ? dest_pos[c0 + k] : -1;
      wt[k] = (k < K) ? (WEIGHTED ? topk_w[c0 + k] : 1.0f) : 0.0f;
    }
    u32x4 *o = out + (size_t)s * vec_per_row;
    for (int base = blockIdx.y * kChunk; base < vec_per_row; base += gridDim.y * kChunk) {
#pragma unroll
      for (int u = 0; u < kCombU; ++u) {
        const int v = base + u * T + threadIdx.x;
        if (v >= vec_per_row) break;
        u32x4 t[kMaxKUnrolled];
#pragma unroll
        for (int k = 0; k < kMaxKUnrolled; ++k)
          if (dst[k] >= 0) t[k] = __builtin_nontemporal_load(y_all + (size_t)dst[k] * vec_per_row + v);
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < kMaxKUnrolled; ++k)
          if (dst[k] >= 0) fma_row16<BF16>(acc, wt[k], t[k]);
        __builtin_nontemporal_store(round_row16<BF16>(acc), o + v);
      }
    }
  }
}

// Generic-K combine for K > kMaxKUnrolled: same arithmetic and order, one k at a time.
template <bool BF16, bool WEIGHTED = true>
__global__ __launch_bounds__(kCombMaxThreads) void k_combine_anyk(const u32x4 *__restrict__ y_all,
                                                             const int32_t *__restrict__ dest_pos,
                                                             const float *__restrict__ topk_w,
                                                             u32x4 *__restrict__ out, int S,
                                                             int K, int rank, int vec_per_row) {
  const int T = blockDim.x, kChunk = T * kCombU;
  for (int s = blockIdx.x; s < S; s += gridDim.x) {
    const size_t c0 = ((size_t)rank * S + s) * K;
    u32x4 *o = out + (size_t)s * vec_per_row;
    for (int base = blockIdx.y * kChunk; base < vec_per_row; base += gridDim.y * kChunk) {
      for (int u = 0; u < kCombU; ++u) {
        const int v = base + u * T + threadIdx.x;
        if (v >= vec_per_row) break;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int k = 0; k < K; ++k) {
          const int d = dest_pos[c0 + k];
          if (d < 0) continue;
          fma_row16<BF16>(acc, WEIGHTED ? topk_w[c0 + k] : 1.0f,
                          y_all[(size_t)d * vec_per_row + v]);
        }
        o[v] = round_row16<BF16>(acc);
      }
    }
  }
}

template <bool BF16>
__device__ inline float dot_row16(u32x4 g, u32x4 y, float acc) {
  if (BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc = __builtin_fmaf(bf16_lo(g[q]), bf16_lo(y[q]), acc);
      acc = __builtin_fmaf(bf16_hi(g[q]), bf16_hi(y[q]), acc);
    }
  } else {
    const f32x4 a = __builtin_bit_cast(f32x4, g), b = __builtin_bit_cast(f32x4, y);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_fmaf(a[q], b[q], acc);
  }
  return acc;
}

constexpr int kWgK = 8;  // copies whose gradients one pass over a token's gradient row serves

// dw[s*K + k] = <dout[s], y_all[dest_pos[c]]>, c = (rank*S + s)*K + k (0 where dest_pos < 0).
// grid (tokens); a block reads its token's output-gradient row once per group of kWgK copies
// and each copy's expert-output row once.  Each thread sums its vectors in row order in fp32,
// then a wave butterfly and the block's waves in index order: a fixed summation order, so the
// result is deterministic.
template <bool BF16>
__global__ __launch_bounds__(kRowThreads) void k_combine_wgrad(const u32x4 *__restrict__ y_all,
                                                              const int32_t *__restrict__ dest_pos,
                                                              const u32x4 *__restrict__ dout,
                                                              float *__restrict__ dw, int S, int K,
                                                              int rank, int vec_per_row) {
  __shared__ float part[kRowThreads / kWave][kWgK];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (int s = blockIdx.x; s < S; s += gridDim.x) {
    const size_t c0 = ((size_t)rank * S + s) * K;
    const u32x4 *g = dout + (size_t)s * vec_per_row;
    for (int kb = 0; kb < K; kb += kWgK) {
      int dst[kWgK];
      float acc[kWgK];
#pragma unroll
      for (int k = 0; k < kWgK; ++k) {
        dst[k] = (kb + k < K) ? dest_pos[c0 + kb + k] : -1;
        acc[k] = 0.0f;
      }
      for (int v = threadIdx.x; v < vec_per_row; v += kRowThreads) {
        const u32x4 gv = __builtin_nontemporal_load(g + v);
        u32x4 yv[kWgK];
#pragma unroll
        for (int k = 0; k < kWgK; ++k)
          if (dst[k] >= 0) yv[k] = __builtin_nontemporal_load(y_all + (size_t)dst[k] * vec_per_row + v);
#pragma unroll
        for (int k = 0; k < kWgK; ++k)
          if (dst[k] >= 0) acc[k] = dot_row16<BF16>(gv, yv[k], acc[k]);
      }
#pragma unroll
      for (int k = 0; k < kWgK; ++k) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc[k] += __shfl_xor(acc[k], off, kWave);
      }
      if (lane == 0) {
#pragma unroll
        for (int k = 0; k < kWgK; ++k) part[wid][k] = acc[k];
      }
      __syncthreads();
      if (threadIdx.x < kWgK && kb + (int)threadIdx.x < K) {
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < kRowThreads / kWave; ++w) t += part[w][threadIdx.x];
        dw[(size_t)s * K + kb + threadIdx.x] = t;
      }
      __syncthreads();
    }
  }
}

// Gated-unit backward, elementwise over (gate, up) pairs: with g, u the stored pre-activation
// pair and d the output gradient, dh_gate = d * u * silu'(g), dh_up = d * silu(g), in fp32,
// one rounding.  The arrays are flat (row-major, no padding): output-gradient vector v (8
// bf16 or 4 fp32 pairs) goes with pre-activation vectors 2v and 2v+1.  One-shot grid.
template <bool BF16>
__global__ __launch_bounds__(kRowThreads) void k_swiglu_bwd(const u32x4 *__restrict__ h,
                                                           const u32x4 *__restrict__ dz,
                                                           u32x4 *__restrict__ dh, long long n_vec) {
  constexpr int kChunk = kRowThreads * kStreamU;
  for (long long base = (long long)blockIdx.x * kChunk; base < n_vec;
       base += (long long)gridDim.x * kChunk) {
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const long long v = base + u * kRowThreads + threadIdx.x;
      if (v >= n_vec) break;
      const u32x4 d = dz[v], h0 = h[2 * v], h1 = h[2 * v + 1];
      u32x4 o0, o1;
      if (BF16) {
        // pair q of d (q = 0..7) is (gate, up) = word q of the 16-value h pair h0|h1
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t hw = q < 4 ? h0[q] : h1[q - 4];
          const float g = bf16_lo(hw), up = bf16_hi(hw);
          const float dd = (q & 1) ? bf16_hi(d[q >> 1]) : bf16_lo(d[q >> 1]);
          const float sg = 1.0f / (1.0f + __expf(-g));
          const uint32_t r = pack_bf16x2(dd * up * sg * (1.0f + g * (1.0f - sg)), dd * g * sg);
          if (q < 4) o0[q] = r; else o1[q - 4] = r;
        }
      } else {
        const f32x4 df = __builtin_bit_cast(f32x4, d);
        const f32x4 a = __builtin_bit_cast(f32x4, h0), b = __builtin_bit_cast(f32x4, h1);
        f32x4 r0, r1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float g = q < 2 ? a[2 * q] : b[2 * (q - 2)];
          const float up = q < 2 ? a[2 * q + 1] : b[2 * (q - 2) + 1];
          const float sg = 1.0f / (1.0f + __expf(-g));
          const float dg = df[q] * up * sg * (1.0f + g * (1.0f - sg)), du = df[q] * g * sg;
          if (q < 2) { r0[2 * q] = dg; r0[2 * q + 1] = du; } else { r1[2 * (q - 2)] = dg; r1[2 * (q - 2) + 1] = du; }
        }
        o0 = __builtin_bit_cast(u32x4, r0);
        o1 = __builtin_bit_cast(u32x4, r1);
      }
      __builtin_nontemporal_store(o0, dh + 2 * v);
      __builtin_nontemporal_store(o1, dh + 2 * v + 1);
    }
  }
}

// dw[e] += dw[E+j]; dw[E+j] = 0 for every used slot j of `rank`.  grid (chunks, B);
// a block covers kRowThreads*kStreamU vectors of one slot row.
__global__ __launch_bounds__(kRowThreads) void k_fold(const int32_t *__restrict__ plan,
                                                     f32x4 *__restrict__ dw, int E, int R, int B,
                                                     int rank, long long vec_per_row) {
  constexpr int kChunk = kRowThreads * kStreamU;
  const PlanLayout L(E, R, B);
  const int j = blockIdx.y;
  const int e = plan[L.off_sexp + rank * B + j];
  if (e < 0) return;
  f32x4 *home = dw + (size_t)e * vec_per_row;
  f32x4 *slot = dw + (size_t)(E + j) * vec_per_row;
  for (long long base = (long long)blockIdx.x * kChunk; base < vec_per_row;
       base += (long long)gridDim.x * kChunk) {
    f32x4 a[kStreamU], b[kStreamU];
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const long long v = base + u * kRowThreads + threadIdx.x;
      if (v < vec_per_row) {
        a[u] = home[v];
        b[u] = __builtin_nontemporal_load(slot + v);
      }
    }
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const long long v = base + u * kRowThreads + threadIdx.x;
      if (v < vec_per_row) {
        home[v] = a[u] + b[u];
        __builtin_nontemporal_store((f32x4){0, 0, 0, 0}, slot + v);
      }
    }
  }
}

// w[E+j] = w[e] for every used slot j of `rank`.  grid (chunks, B).
__global__ __launch_bounds__(kRowThreads) void k_prefetch(const int32_t *__restrict__ plan,
                                                         u32x4 *__restrict__ w, int E, int R,
                                                         int B, int rank, long long vec_per_row) {
  constexpr int kChunk = kRowThreads * kStreamU;
  const PlanLayout L(E, R, B);
  const int j = blockIdx.y;
  const int e = plan[L.off_sexp + rank * B + j];
  if (e < 0) return;
  const u32x4 *src = w + (size_t)e * vec_per_row;
  u32x4 *dst = w + (size_t)(E + j) * vec_per_row;
  for (long long base = (long long)blockIdx.x * kChunk; base < vec_per_row;
       base += (long long)gridDim.x * kChunk) {
    u32x4 t[kStreamU];
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const long long v = base + u * kRowThreads + threadIdx.x;
      if (v < vec_per_row) t[u] = __builtin_nontemporal_load(src + v);
    }
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const long long v = base + u * kRowThreads + threadIdx.x;
      if (v < vec_per_row) __builtin_nontemporal_store(t[u], dst + v);
    }
  }
}

static unsigned clamp_grid(long long want, long long cap) {
  return (unsigned)(want < 1 ? 1 : (want < cap ? want : cap));
}

}  // namespace moe

using namespace moe;

static int elem_bytes(moe_dtype t) { return t == MOE_BF16 ? 2 : (t == MOE_F32 ? 4 : 0); }

extern "C" moe_status_t moe_permute(const moe_dims *d, moe_dtype dtype, int64_t width,
                                    const void *x_all, const int32_t *src_flat,
                                    const float *row_scale, void *xp, hipStream_t stream) {
  if (!dims_ok(d) || !x_all || !src_flat || !xp) return MOE_EINVAL;
  const int eb = elem_bytes(dtype);
  if (!eb || width <= 0 || (width * eb) % 16 != 0 || width * eb / 16 > INT32_MAX) return MOE_EINVAL;
  const int SK = d->S * d->K;
  const int vec = (int)(width * eb / 16);
  // One block per row chunk; the block is as wide as the row (rounded to a wave) up to
  // kPermMaxThreads, one 16-byte vector per thread.
  const int threads = (int)(vec < kPermMaxThreads ? ((vec + kWave - 1) / kWave) * kWave
                                                  : kPermMaxThreads);
  const unsigned gy = clamp_grid(ceil_div(vec, threads), kMaxGridY);
  if (row_scale)
    hipLaunchKernelGGL(k_permute<true>, dim3(clamp_grid(ceil_div(SK, kPermRows<true>), kMaxGridX), gy),
                       dim3(threads), 0, stream, (const u32x4 *)x_all, src_flat, row_scale,
                       (u32x4 *)xp, SK, d->K, vec, dtype == MOE_BF16);
  else
    hipLaunchKernelGGL(k_permute<false>, dim3(clamp_grid(ceil_div(SK, kPermRows<false>), kMaxGridX), gy),
                       dim3(threads), 0, stream, (const u32x4 *)x_all, src_flat, row_scale,
                       (u32x4 *)xp, SK, d->K, vec, dtype == MOE_BF16);
  return launch_status();
}

extern "C" moe_status_t moe_combine(const moe_dims *d, moe_dtype dtype, int64_t width,
                                    int32_t rank, const void *y_all, const int32_t *dest_pos,
                                    const float *topk_w, void *out, hipStream_t stream) {
  if (!dims_ok(d) || !y_all || !dest_pos || !topk_w || !out) return MOE_EINVAL;
  if (rank < 0 || rank >= d->R) return MOE_EINVAL;
  const int eb = elem_bytes(dtype);
  if (!eb || width <= 0 || (width * eb) % 16 != 0 || width * eb / 16 > INT32_MAX) return MOE_EINVAL;
  const int vec = (int)(width * eb / 16);
  const int threads = comb_threads(vec);
  const dim3 grid(clamp_grid(d->S, kMaxGridX),
                  clamp_grid(ceil_div(vec, threads * kCombU), kMaxGridY));
  const bool bf = dtype == MOE_BF16;
  if (d->K <= kMaxKUnrolled) {
    if (bf)
      hipLaunchKernelGGL(k_combine<true>, grid, dim3(threads), 0, stream,
                         (const u32x4 *)y_all, dest_pos, topk_w, (u32x4 *)out, d->S, d->K, rank,
                         vec);
    else
      hipLaunchKernelGGL(k_combine<false>, grid, dim3(threads), 0, stream,
                         (const u32x4 *)y_all, dest_pos, topk_w, (u32x4 *)out, d->S, d->K, rank,
                         vec);
  } else {
    if (bf)
      hipLaunchKernelGGL(k_combine_anyk<true>, grid, dim3(threads), 0, stream,
                         (const u32x4 *)y_all, dest_pos, topk_w, (u32x4 *)out, d->S, d->K, rank,
                         vec);
    else
      hipLaunchKernelGGL(k_combine_anyk<false>, grid, dim3(threads), 0, stream,
                         (const u32x4 *)y_all, dest_pos, topk_w, (u32x4 *)out, d->S, d->K, rank,
                         vec);
  }
  return launch_status();
}

extern "C" moe_status_t moe_unpermute_reduce(const moe_dims *d, moe_dtype dtype, int64_t width,
                                             int32_t rank, const void *dxp_all,
                                             const int32_t *dest_pos, void *dx,
                                             hipStream_t stream) {
  if (!dims_ok(d) || !dxp_all || !dest_pos || !dx) return MOE_EINVAL;
  if (rank < 0 || rank >= d->R) return MOE_EINVAL;
  const int eb = elem_bytes(dtype);
  if (!eb || width <= 0 || (width * eb) % 16 != 0 || width * eb / 16 > INT32_MAX) return MOE_EINVAL;
  const int vec = (int)(width * eb / 16);
  const int threads = comb_threads(vec);
  const dim3 grid(clamp_grid(d->S, kMaxGridX),
                  clamp_grid(ceil_div(vec, threads * kCombU), kMaxGridY));
  const bool bf = dtype == MOE_BF16;
  const u32x4 *src = (const u32x4 *)dxp_all;
  if (d->K <= kMaxKUnrolled) {
    if (bf)
      hipLaunchKernelGGL((k_combine<true, false>), grid, dim3(threads), 0, stream, src,
                         dest_pos, nullptr, (u32x4 *)dx, d->S, d->K, rank, vec);
    else
      hipLaunchKernelGGL((k_combine<false, false>), grid, dim3(threads), 0, stream, src,
                         dest_pos, nullptr, (u32x4 *)dx, d->S, d->K, rank, vec);
  } else {
    if (bf)
      hipLaunchKernelGGL((k_combine_anyk<true, false>), grid, dim3(threads), 0, stream, src,
                         dest_pos, nullptr, (u32x4 *)dx, d->S, d->K, rank, vec);
    else
      hipLaunchKernelGGL((k_combine_anyk<false, false>), grid, dim3(threads), 0, stream, src,
                         dest_pos, nullptr, (u32x4 *)dx, d->S, d->K, rank, vec);
  }
  return launch_status();
}

extern "C" moe_status_t moe_combine_weight_grad(const moe_dims *d, moe_dtype dtype, int64_t width,
                                                int32_t rank, const void *y_all,
                                                const int32_t *dest_pos, const void *dout,
                                                float *dw, hipStream_t stream) {
  if (!dims_ok(d) || !y_all || !dest_pos || !dout || !dw) return MOE_EINVAL;
  if (rank < 0 || rank >= d->R) return MOE_EINVAL;
  const int eb = elem_bytes(dtype);
  if (!eb || width <= 0 || (width * eb) % 16 != 0 || width * eb / 16 > INT32_MAX) return MOE_EINVAL;
  const int vec = (int)(width * eb / 16);
  const dim3 grid(clamp_grid(d->S, kMaxGridX));
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(k_combine_wgrad<true>, grid, dim3(kRowThreads), 0, stream,
                       (const u32x4 *)y_all, dest_pos, (const u32x4 *)dout, dw, d->S, d->K, rank,
                       vec);
  else
    hipLaunchKernelGGL(k_combine_wgrad<false>, grid, dim3(kRowThreads), 0, stream,
                       (const u32x4 *)y_all, dest_pos, (const u32x4 *)dout, dw, d->S, d->K, rank,
                       vec);
  return launch_status();
}

extern "C" moe_status_t moe_replica_grad_fold(const moe_dims *d, int32_t rank,
                                              const int32_t *plan, float *dw, int64_t row_elems,
                                              hipStream_t stream) {
  if (!dims_ok(d) || !plan || !dw || row_elems <= 0 || row_elems % 4 != 0) return MOE_EINVAL;
  if (rank < 0 || rank >= d->R) return MOE_EINVAL;
  if (d->B == 0) return MOE_OK;
  const long long vec = row_elems / 4;
  const dim3 grid(clamp_grid((vec + kRowThreads * kStreamU - 1) / (kRowThreads * kStreamU),
                             kMaxGridX),
                  d->B);
  hipLaunchKernelGGL(k_fold, grid, dim3(kRowThreads), 0, stream, plan, (f32x4 *)dw, d->E, d->R,
                     d->B, rank, vec);
  return launch_status();
}

extern "C" moe_status_t moe_prefetch(const moe_dims *d, int32_t rank, const int32_t *plan,
                                     void *w, int64_t row_bytes, hipStream_t stream) {
  if (!dims_ok(d) || !plan || !w || row_bytes <= 0 || row_bytes % 16 != 0) return MOE_EINVAL;
  if (rank < 0 || rank >= d->R) return MOE_EINVAL;
  if (d->B == 0) return MOE_OK;
  const long long vec = row_bytes / 16;
  const dim3 grid(clamp_grid((vec + kRowThreads * kStreamU - 1) / (kRowThreads * kStreamU),
                             kMaxGridX),
                  d->B);
  hipLaunchKernelGGL(k_prefetch, grid, dim3(kRowThreads), 0, stream, plan, (u32x4 *)w, d->E,
                     d->R, d->B, rank, vec);
  return launch_status();
}

extern "C" moe_status_t moe_swiglu_backward(moe_dtype dtype, int64_t rows, int64_t n_pairs,
                                            const void *h, const void *dz, void *dh,
                                            hipStream_t stream) {
  if (!h || !dz || !dh || rows < 0 || n_pairs <= 0) return MOE_EINVAL;
  const int eb = elem_bytes(dtype);
  if (!eb || (n_pairs * eb) % 16 != 0) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  const long long n_vec = rows * n_pairs * eb / 16;
  const dim3 grid(clamp_grid((n_vec + kRowThreads * kStreamU - 1) / (kRowThreads * kStreamU),
                             kMaxGridX));
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(k_swiglu_bwd<true>, grid, dim3(kRowThreads), 0, stream, (const u32x4 *)h,
                       (const u32x4 *)dz, (u32x4 *)dh, n_vec);
  else
    hipLaunchKernelGGL(k_swiglu_bwd<false>, grid, dim3(kRowThreads), 0, stream,
                       (const u32x4 *)h, (const u32x4 *)dz, (u32x4 *)dh, n_vec);
  return launch_status();
}
