// Row-streaming kernels: gather-permute, weighted combine, replica-gradient
// fold and slot prefetch.  All are HBM-bound; each moves whole rows with
// 16-byte vector loads/stores, one wavefront per row, several rows in flight
// per lane.
//
// Pages: moses-y.github.io "MoonEP", "What This Does" and "Real-World Use";
// findrepo.work "MoonEP" card, "Strengths" (fused permute / unpermute);
// ainovat.com "Moonshot AI Open-Sources MoonEP", mechanism paragraph
// (replica weights fetched ahead, replica gradients returned home).
#include "common.hpp"

namespace moe {

constexpr int kRowThreads = 256;
constexpr int kUnroll = 4;

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

// xp[i] = x_all[src_flat[i] / K] (optionally * row_scale[src]); one wave per row.
template <bool SCALED>
__global__ __launch_bounds__(kRowThreads) void k_permute(const u32x4 *__restrict__ x_all,
                                                        const int32_t *__restrict__ src_flat,
                                                        const float *__restrict__ scale,
                                                        u32x4 *__restrict__ xp, int SK, int K,
                                                        int vec_per_row, int bf16) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * kRowThreads + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * kRowThreads) >> 6;
  for (int i = wave; i < SK; i += nwaves) {
    const int src = src_flat[i];
    u32x4 *dst = xp + (size_t)i * vec_per_row;
    if (src < 0) {
      for (int v = lane; v < vec_per_row; v += kWave) dst[v] = (u32x4){0, 0, 0, 0};
      continue;
    }
    const u32x4 *row = x_all + (size_t)(src / K) * vec_per_row;
    const float w = SCALED ? scale[src] : 1.0f;
    int v = lane;
    for (; v + (kUnroll - 1) * kWave < vec_per_row; v += kUnroll * kWave) {
      u32x4 t[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) t[u] = __builtin_nontemporal_load(row + v + u * kWave);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const u32x4 o = SCALED ? scale_row16(t[u], w, bf16) : t[u];
        __builtin_nontemporal_store(o, dst + v + u * kWave);
      }
    }
    for (; v < vec_per_row; v += kWave) {
      const u32x4 t = __builtin_nontemporal_load(row + v);
      __builtin_nontemporal_store(SCALED ? scale_row16(t, w, bf16) : t, dst + v);
    }
  }
}

constexpr int kMaxKUnrolled = 16;

// out[s] = sum_k w[c] * y_all[dest_pos[c]], c = (rank*S + s)*K + k; one wave per token.
template <bool BF16>
__global__ __launch_bounds__(kRowThreads) void k_combine(const u32x4 *__restrict__ y_all,
                                                        const int32_t *__restrict__ dest_pos,
                                                        const float *__restrict__ topk_w,
                                                        u32x4 *__restrict__ out, int S, int K,
                                                        int rank, int vec_per_row) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * kRowThreads + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * kRowThreads) >> 6;
  for (int s = wave; s < S; s += nwaves) {
    const size_t c0 = ((size_t)rank * S + s) * K;
    int dst[kMaxKUnrolled];
    float wt[kMaxKUnrolled];
#pragma unroll
    for (int k = 0; k < kMaxKUnrolled; ++k) {
      dst[k] = (k < K) ? dest_pos[c0 + k] : -1;
      wt[k] = (k < K) ? topk_w[c0 + k] : 0.0f;
    }
    u32x4 *o = out + (size_t)s * vec_per_row;
    for (int v = lane; v < vec_per_row; v += kWave) {
      u32x4 t[kMaxKUnrolled];
#pragma unroll
      for (int k = 0; k < kMaxKUnrolled; ++k)
        if (dst[k] >= 0) t[k] = y_all[(size_t)dst[k] * vec_per_row + v];
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < kMaxKUnrolled; ++k) {
        if (dst[k] < 0) continue;
        if (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] = __builtin_fmaf(wt[k], bf16_lo(t[k][q]), acc[2 * q]);
            acc[2 * q + 1] = __builtin_fmaf(wt[k], bf16_hi(t[k][q]), acc[2 * q + 1]);
          }
        } else {
          const f32x4 f = __builtin_bit_cast(f32x4, t[k]);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(wt[k], f[q], acc[q]);
        }
      }
      u32x4 r;
      if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      } else {
        r = __builtin_bit_cast(u32x4, (f32x4){acc[0], acc[1], acc[2], acc[3]});
      }
      __builtin_nontemporal_store(r, o + v);
    }
  }
}

// Generic-K combine for K > kMaxKUnrolled: same arithmetic, loads one k at a time.
template <bool BF16>
__global__ __launch_bounds__(kRowThreads) void k_combine_anyk(const u32x4 *__restrict__ y_all,
                                                             const int32_t *__restrict__ dest_pos,
                                                             const float *__restrict__ topk_w,
                                                             u32x4 *__restrict__ out, int S,
                                                             int K, int rank, int vec_per_row) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * kRowThreads + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * kRowThreads) >> 6;
  for (int s = wave; s < S; s += nwaves) {
    const size_t c0 = ((size_t)rank * S + s) * K;
    u32x4 *o = out + (size_t)s * vec_per_row;
    for (int v = lane; v < vec_per_row; v += kWave) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int k = 0; k < K; ++k) {
        const int d = dest_pos[c0 + k];
        if (d < 0) continue;
        const float w = topk_w[c0 + k];
        const u32x4 t = y_all[(size_t)d * vec_per_row + v];
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
      u32x4 r;
      if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      } else {
        r = __builtin_bit_cast(u32x4, (f32x4){acc[0], acc[1], acc[2], acc[3]});
      }
      o[v] = r;
    }
  }
}

// dw[e] += dw[E+j]; dw[E+j] = 0 for every used slot j of `rank`.  grid (blocks, B).
__global__ __launch_bounds__(kRowThreads) void k_fold(const int32_t *__restrict__ plan,
                                                     f32x4 *__restrict__ dw, int E, int R, int B,
                                                     int rank, long long vec_per_row) {
  const PlanLayout L(E, R, B);
  const int j = blockIdx.y;
  const int e = plan[L.off_sexp + rank * B + j];
  if (e < 0) return;
  f32x4 *home = dw + (size_t)e * vec_per_row;
  f32x4 *slot = dw + (size_t)(E + j) * vec_per_row;
  const long long stride = (long long)gridDim.x * kRowThreads;
  long long v = (long long)blockIdx.x * kRowThreads + threadIdx.x;
  for (; v + stride < vec_per_row; v += 2 * stride) {
    const f32x4 a0 = home[v], b0 = __builtin_nontemporal_load(slot + v);
    const f32x4 a1 = home[v + stride], b1 = __builtin_nontemporal_load(slot + v + stride);
    home[v] = a0 + b0;
    home[v + stride] = a1 + b1;
    __builtin_nontemporal_store((f32x4){0, 0, 0, 0}, slot + v);
    __builtin_nontemporal_store((f32x4){0, 0, 0, 0}, slot + v + stride);
  }
  for (; v < vec_per_row; v += stride) {
    home[v] = home[v] + slot[v];
    slot[v] = (f32x4){0, 0, 0, 0};
  }
}

// w[E+j] = w[e] for every used slot j of `rank`.  grid (blocks, B).
__global__ __launch_bounds__(kRowThreads) void k_prefetch(const int32_t *__restrict__ plan,
                                                         u32x4 *__restrict__ w, int E, int R,
                                                         int B, int rank, long long vec_per_row) {
  const PlanLayout L(E, R, B);
  const int j = blockIdx.y;
  const int e = plan[L.off_sexp + rank * B + j];
  if (e < 0) return;
  const u32x4 *src = w + (size_t)e * vec_per_row;
  u32x4 *dst = w + (size_t)(E + j) * vec_per_row;
  const long long stride = (long long)gridDim.x * kRowThreads;
  for (long long v = (long long)blockIdx.x * kRowThreads + threadIdx.x; v < vec_per_row;
       v += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + v), dst + v);
}

static int row_grid(long long rows, int waves_per_block = kRowThreads / kWave) {
  const long long want = (rows + waves_per_block - 1) / waves_per_block;
  const long long cap = (long long)device_cu_count() * 16;
  return (int)(want < cap ? (want < 1 ? 1 : want) : cap);
}

}  // namespace moe

using namespace moe;

static int elem_bytes(moe_dtype t) { return t == MOE_BF16 ? 2 : (t == MOE_F32 ? 4 : 0); }

extern "C" moe_status_t moe_permute(const moe_dims *d, moe_dtype dtype, int64_t width,
                                    const void *x_all, const int32_t *src_flat,
                                    const float *row_scale, void *xp, hipStream_t stream) {
  if (!dims_ok(d) || !x_all || !src_flat || !xp) return MOE_EINVAL;
  const int eb = elem_bytes(dtype);
  if (!eb || width <= 0 || (width * eb) % 16 != 0) return MOE_EINVAL;
  const int SK = d->S * d->K;
  const int vec = (int)(width * eb / 16);
  const int grid = row_grid(SK);
  if (row_scale)
    hipLaunchKernelGGL(k_permute<true>, dim3(grid), dim3(kRowThreads), 0, stream,
                       (const u32x4 *)x_all, src_flat, row_scale, (u32x4 *)xp, SK, d->K, vec,
                       dtype == MOE_BF16);
  else
    hipLaunchKernelGGL(k_permute<false>, dim3(grid), dim3(kRowThreads), 0, stream,
                       (const u32x4 *)x_all, src_flat, row_scale, (u32x4 *)xp, SK, d->K, vec,
                       dtype == MOE_BF16);
  return launch_status();
}

extern "C" moe_status_t moe_combine(const moe_dims *d, moe_dtype dtype, int64_t width,
                                    int32_t rank, const void *y_all, const int32_t *dest_pos,
                                    const float *topk_w, void *out, hipStream_t stream) {
  if (!dims_ok(d) || !y_all || !dest_pos || !topk_w || !out) return MOE_EINVAL;
  if (rank < 0 || rank >= d->R) return MOE_EINVAL;
  const int eb = elem_bytes(dtype);
  if (!eb || width <= 0 || (width * eb) % 16 != 0) return MOE_EINVAL;
  const int vec = (int)(width * eb / 16);
  const int grid = row_grid(d->S);
  const bool bf = dtype == MOE_BF16;
  if (d->K <= kMaxKUnrolled) {
    if (bf)
      hipLaunchKernelGGL(k_combine<true>, dim3(grid), dim3(kRowThreads), 0, stream,
                         (const u32x4 *)y_all, dest_pos, topk_w, (u32x4 *)out, d->S, d->K, rank,
                         vec);
    else
      hipLaunchKernelGGL(k_combine<false>, dim3(grid), dim3(kRowThreads), 0, stream,
                         (const u32x4 *)y_all, dest_pos, topk_w, (u32x4 *)out, d->S, d->K, rank,
                         vec);
  } else {
    if (bf)
      hipLaunchKernelGGL(k_combine_anyk<true>, dim3(grid), dim3(kRowThreads), 0, stream,
                         (const u32x4 *)y_all, dest_pos, topk_w, (u32x4 *)out, d->S, d->K, rank,
                         vec);
    else
      hipLaunchKernelGGL(k_combine_anyk<false>, dim3(grid), dim3(kRowThreads), 0, stream,
                         (const u32x4 *)y_all, dest_pos, topk_w, (u32x4 *)out, d->S, d->K, rank,
                         vec);
  }
  return launch_status();
}

extern "C" moe_status_t moe_replica_grad_fold(const moe_dims *d, int32_t rank,
                                              const int32_t *plan, float *dw, int64_t row_elems,
                                              hipStream_t stream) {
  if (!dims_ok(d) || !plan || !dw || row_elems <= 0 || row_elems % 4 != 0) return MOE_EINVAL;
  if (rank < 0 || rank >= d->R) return MOE_EINVAL;
  if (d->B == 0) return MOE_OK;
  const long long vec = row_elems / 4;
  long long bx = (vec + kRowThreads * 2 - 1) / (kRowThreads * 2);
  const long long cap = (long long)device_cu_count() * 8;
  if (bx > cap) bx = cap;
  hipLaunchKernelGGL(k_fold, dim3((unsigned)bx, d->B), dim3(kRowThreads), 0, stream, plan,
                     (f32x4 *)dw, d->E, d->R, d->B, rank, vec);
  return launch_status();
}

extern "C" moe_status_t moe_prefetch(const moe_dims *d, int32_t rank, const int32_t *plan,
                                     void *w, int64_t row_bytes, hipStream_t stream) {
  if (!dims_ok(d) || !plan || !w || row_bytes <= 0 || row_bytes % 16 != 0) return MOE_EINVAL;
  if (rank < 0 || rank >= d->R) return MOE_EINVAL;
  if (d->B == 0) return MOE_OK;
  const long long vec = row_bytes / 16;
  long long bx = (vec + kRowThreads - 1) / kRowThreads;
  const long long cap = (long long)device_cu_count() * 8;
  if (bx > cap) bx = cap;
  hipLaunchKernelGGL(k_prefetch, dim3((unsigned)bx, d->B), dim3(kRowThreads), 0, stream, plan,
                     (u32x4 *)w, d->E, d->R, d->B, rank, vec);
  return launch_status();
}
