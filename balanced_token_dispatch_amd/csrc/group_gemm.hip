// moe_group_gemm: grouped GEMM over one contiguous [G, Kd, N] weight tensor,
// groups addressed purely by row index, segments given by cu_seqlens.
//
// Pages: ainovat.com "Moonshot AI Open-Sources MoonEP", contract paragraph
// (the group GEMM consumes a single [E+B, H, H'] weight tensor and the
// planner's cu_seqlens selects the active rows) and contiguity paragraph
// (experts are addressed by row index, so the tensor must be contiguous).
//
// bf16 path (MFMA, gfx950):
//   * persistent grid of one 256-thread workgroup per CU; every workgroup
//     rebuilds the tile table from cu_seqlens in LDS (no host sync, the
//     grid is sized from the machine, not from the routing);
//   * 256x256 output tile, K step 64, 4 waves in 2x2, each wave 128x128 as
//     4x4 v_mfma_f32_32x32x16_bf16 blocks (fp32 accumulators);
//   * operands staged global -> registers -> LDS, double-buffered, one
//     barrier per K step, next tile's global loads in flight during the
//     MFMAs; an operand whose contraction index is strided in memory (the
//     weight in FWD, both operands in WGRAD) is transposed 8x8 in registers
//     on its way to LDS so every LDS row holds contiguous contraction values;
//   * the MFMA is issued as (weight-side x activation-side) so each lane
//     ends with 4 consecutive output columns: 8-byte bf16 / 16-byte fp32
//     stores;
//   * blockIdx is remapped so the 32 workgroups of one XCD work on
//     neighbouring tiles (shared weight and activation panels in that XCD's
//     L2); tiles are walked in groups of 8 row-tiles.
// fp32 path: plain vector-ALU kernels (small shapes only).
#include "common.hpp"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGemmThreads = 256;
constexpr int LDS_STRIDE = BK + 8;            // bf16 elements per LDS row (144 B)
constexpr int TILE_ELEMS = BM * LDS_STRIDE;   // one operand tile (BM == BN)
constexpr int kMaxG = 1088;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

// Buffer resource over [base, base + bytes): loads past the end return zero.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, long long bytes) {
  const int n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}
constexpr int kOOB = 0x7FFFFFF0;  // an offset past every resource: the load returns zero

// Contraction-contiguous operand: row r, contraction c at base[r*ld + c].
// Each thread moves 8 chunks of 8 elements: chunk q = tid + 256*u -> row q/8, col (q%8)*8.
struct ContigLoad {
  u32x4 v[8];
  __device__ void load(__amdgpu_buffer_rsrc_t rs, int ld, int row_lim, int c0, int c_lim) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int q = threadIdx.x + kGemmThreads * u;
      const int r = q >> 3, c = c0 + (q & 7) * 8;
      const int off = (r < row_lim && c < c_lim) ? (r * ld + c) * 2 : kOOB;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    }
  }
  __device__ void store(uint16_t *lds) const {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int q = threadIdx.x + kGemmThreads * u;
      *(u32x4 *)(lds + (q >> 3) * LDS_STRIDE + (q & 7) * 8) = v[u];
    }
  }
};

// Contraction-strided operand: row r, contraction c at base[c*ld + r].
// Each thread moves one 8x8 block: contraction rows cb*8..+8, rows ib*8..+8, and
// transposes it in registers.  cb = tid%8, ib = tid/8: a load instruction reads 128
// contiguous bytes per contraction row, and the 16 lanes of each LDS write group hit
// 8 column chunks x 2 row parities = 16 distinct bank quads (rows are 144 B apart).
struct StridedLoad {
  u32x4 v[8];  // v[kk] = 8 row values at contraction index cb*8+kk
  __device__ void load(__amdgpu_buffer_rsrc_t rs, int ld, int row_lim, int c0, int c_lim) {
    const int cb = threadIdx.x & 7, ib = threadIdx.x >> 3;
    const int r = ib * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int c = c0 + cb * 8 + kk;
      const int off = (r < row_lim && c < c_lim) ? (c * ld + r) * 2 : kOOB;
      v[kk] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    }
  }
  __device__ void store(uint16_t *lds) const {
    const int cb = threadIdx.x & 7, ib = threadIdx.x >> 3;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      // row ib*8+rr: contraction values cb*8+0..7 = element rr of v[0..7]
      u32x4 o;
      const int half = rr & 1, w = rr >> 1;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a = v[2 * p][w], b = v[2 * p + 1][w];
        o[p] = half ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
      }
      *(u32x4 *)(lds + (ib * 8 + rr) * LDS_STRIDE + cb * 8) = o;
    }
  }
};

template <bool CONTIG>
struct Loader;
template <>
struct Loader<true> { typedef ContigLoad T; };
template <>
struct Loader<false> { typedef StridedLoad T; };

struct Frags {
  bf16x8 a[4], b[4];
};

__device__ inline void read_frags(Frags &f, const uint16_t *As, const uint16_t *Bs, int wi, int wj,
                                  int lane, int ks) {
  const int col = ks * 16 + (lane >> 5) * 8;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f.a[t] = __builtin_bit_cast(bf16x8,
                                *(const u32x4 *)(As + (wi + t * 32 + (lane & 31)) * LDS_STRIDE + col));
    f.b[t] = __builtin_bit_cast(bf16x8,
                                *(const u32x4 *)(Bs + (wj + t * 32 + (lane & 31)) * LDS_STRIDE + col));
  }
}

__device__ inline void mma16(f32x16 (&acc)[4][4], const Frags &f) {
#pragma unroll
  for (int tm = 0; tm < 4; ++tm)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
      acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[tn], f.a[tm], acc[tm][tn], 0, 0, 0);
}

// One 256x256 output tile: out_tile[i][j] = sum_c Aop(i, c) * Bop(j, c).
// Aop rows i (activations or x^T), Bop rows j (weights or dy^T).  Pipeline per K step kt:
// fragments of step kt come from LDS buffer kt&1 (double-buffered in registers across the
// four 16-wide MFMA sub-steps); meanwhile tile kt+1, loaded into registers during step
// kt-1, is written to the other LDS buffer and tile kt+2 is requested from memory.
template <bool A_CONTIG, bool B_CONTIG>
__device__ inline void tile_mma(uint16_t *lds, __amdgpu_buffer_rsrc_t ra, int lda, int a_rows,
                                __amdgpu_buffer_rsrc_t rb, int ldb, int b_rows, int c_len,
                                f32x16 (&acc)[4][4]) {
  typename Loader<A_CONTIG>::T la;
  typename Loader<B_CONTIG>::T lb;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wi = (wid >> 1) * 128, wj = (wid & 1) * 128;
  const int nk = (c_len + BK - 1) / BK;

#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = (f32x16){};

  la.load(ra, lda, a_rows, 0, c_len);
  lb.load(rb, ldb, b_rows, 0, c_len);
  la.store(lds);
  lb.store(lds + TILE_ELEMS);
  if (nk > 1) {
    la.load(ra, lda, a_rows, BK, c_len);
    lb.load(rb, ldb, b_rows, BK, c_len);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const uint16_t *As = lds + (kt & 1) * 2 * TILE_ELEMS;
    const uint16_t *Bs = As + TILE_ELEMS;
    uint16_t *An = lds + ((kt + 1) & 1) * 2 * TILE_ELEMS;
    Frags f0, f1;
    read_frags(f0, As, Bs, wi, wj, lane, 0);
    if (kt + 1 < nk) {
      la.store(An);
      lb.store(An + TILE_ELEMS);
      if (kt + 2 < nk) {
        la.load(ra, lda, a_rows, (kt + 2) * BK, c_len);
        lb.load(rb, ldb, b_rows, (kt + 2) * BK, c_len);
      }
    }
    read_frags(f1, As, Bs, wi, wj, lane, 1);
    // keep each sub-step's fragment reads ahead of the previous sub-step's MFMAs
    __builtin_amdgcn_sched_barrier(0);
    mma16(acc, f0);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(f0, As, Bs, wi, wj, lane, 2);
    __builtin_amdgcn_sched_barrier(0);
    mma16(acc, f1);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(f1, As, Bs, wi, wj, lane, 3);
    __builtin_amdgcn_sched_barrier(0);
    mma16(acc, f0);
    __builtin_amdgcn_sched_barrier(0);
    mma16(acc, f1);
    __syncthreads();
  }
}

// Decode a tile index into (row tile, col tile) walking groups of kGroupM row tiles.
__device__ inline void swizzle(int t, int n_rt, int n_ct, int *rt, int *ct) {
  const int per_group = kGroupM * n_ct;
  const int g = t / per_group;
  const int r = t - g * per_group;
  const int gm = min(kGroupM, n_rt - g * kGroupM);
  *rt = g * kGroupM + r % gm;
  *ct = r / gm;
}

__device__ inline int logical_block() {
  // workgroups are dealt round-robin to the XCDs; give each XCD a contiguous range
  const int b = blockIdx.x, n = gridDim.x;
  if (n % kXcds) return b;
  return (b % kXcds) * (n / kXcds) + b / kXcds;
}

// Segment table: sCu[rho] (clamped to [0, M_total]) and sStart[rho] = first row tile of rho.
__device__ inline int build_tiles(const int32_t *cu, int G, int M_total, int *sCu, int *sStart,
                                  bool wgrad) {
  __shared__ int tmp[4];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int i = tid; i <= G; i += kGemmThreads) sCu[i] = min(max(cu[i], 0), M_total);
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < G; base += kGemmThreads) {
    const int rho = base + tid;
    int v = 0;
    if (rho < G) {
      const int n = sCu[rho + 1] - sCu[rho];
      v = n > 0 ? (wgrad ? 1 : (n + BM - 1) / BM) : 0;
    }
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) tmp[wid] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      before += w < wid ? tmp[w] : 0;
      tot += tmp[w];
    }
    const int carry = carry_s;
    if (rho < G) sStart[rho] = carry + before + x - v;
    __syncthreads();
    if (tid == 0) carry_s = carry + tot;
    __syncthreads();
  }
  const int total = carry_s;
  if (tid == 0) sStart[G] = total;
  __syncthreads();
  return total;
}

// last rho with sStart[rho] <= t (the segment owning row tile t)
__device__ inline int find_seg(const int *sStart, int G, int t) {
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (sStart[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

template <int OP>
__global__ __launch_bounds__(kGemmThreads, 1) void k_ggemm_bf16(
    const uint16_t *__restrict__ a, const uint16_t *__restrict__ b,
    const int32_t *__restrict__ cu, void *__restrict__ out, int G, int M_total, int Kd, int N) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ int sCu[kMaxG + 1], sStart[kMaxG + 1];
  const bool wgrad = OP == MOE_GEMM_WGRAD;
  const int n_rt_total = build_tiles(cu, G, M_total, sCu, sStart, wgrad);
  // FWD: i = rows, j = n in [0,N), c = kd.  DGRAD: i = rows, j = kd, c = n.
  // WGRAD: i = kd, j = n, c = rows of the segment (per active segment: n_it x n_jt tiles).
  const int ncols = OP == MOE_GEMM_DGRAD ? Kd : N;
  const int n_ct = (ncols + BN - 1) / BN;
  const int n_it = (Kd + BM - 1) / BM;
  const long long total = wgrad ? (long long)n_rt_total * n_it * n_ct : (long long)n_rt_total * n_ct;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wi = (wid >> 1) * 128, wj = (wid & 1) * 128;

  for (long long t = logical_block(); t < total; t += gridDim.x) {
    f32x16 acc[4][4];
    if (!wgrad) {
      int rt, ct;
      swizzle((int)t, n_rt_total, n_ct, &rt, &ct);
      const int rho = find_seg(sStart, G, rt);
      const int m0 = sCu[rho] + (rt - sStart[rho]) * BM;
      const int rows = min(BM, sCu[rho + 1] - m0);
      const int j0 = ct * BN;
      const uint16_t *w = b + (size_t)rho * Kd * N;
      if (OP == MOE_GEMM_FWD)
        tile_mma<true, false>(lds, make_rsrc(a + (size_t)m0 * Kd, (long long)rows * Kd * 2), Kd,
                              rows, make_rsrc(w + j0, ((long long)Kd * N - j0) * 2), N, N - j0, Kd,
                              acc);
      else
        tile_mma<true, true>(lds, make_rsrc(a + (size_t)m0 * N, (long long)rows * N * 2), N, rows,
                             make_rsrc(w + (size_t)j0 * N, (long long)(Kd - j0) * N * 2), N,
                             Kd - j0, N, acc);
      uint16_t *o = (uint16_t *)out + (size_t)m0 * ncols + j0;
#pragma unroll
      for (int tm = 0; tm < 4; ++tm) {
        const int i = wi + tm * 32 + (lane & 31);
        if (i >= rows) continue;
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int j = wj + tn * 32 + g * 8 + (lane >> 5) * 4;
            if (j0 + j < ncols) {
              const f32x16 &c = acc[tm][tn];
              uint2 v;
              v.x = pack_bf16x2(c[4 * g + 0], c[4 * g + 1]);
              v.y = pack_bf16x2(c[4 * g + 2], c[4 * g + 3]);
              *(uint2 *)(o + (size_t)i * ncols + j) = v;
            }
          }
      }
    } else {
      const int per_seg = n_it * n_ct;
      const int sidx = (int)(t / per_seg);
      int it, ct;
      swizzle((int)(t - (long long)sidx * per_seg), n_it, n_ct, &it, &ct);
      const int rho = find_seg(sStart, G, sidx);
      const int m0 = sCu[rho], len = sCu[rho + 1] - m0;
      const int i0 = it * BM, j0 = ct * BN;
      tile_mma<false, false>(lds, make_rsrc(a + (size_t)m0 * Kd + i0, ((long long)len * Kd - i0) * 2),
                             Kd, Kd - i0,
                             make_rsrc(b + (size_t)m0 * N + j0, ((long long)len * N - j0) * 2), N,
                             N - j0, len, acc);
      float *o = (float *)out + ((size_t)rho * Kd + i0) * N + j0;
#pragma unroll
      for (int tm = 0; tm < 4; ++tm) {
        const int i = wi + tm * 32 + (lane & 31);
        if (i0 + i >= Kd) continue;
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int j = wj + tn * 32 + g * 8 + (lane >> 5) * 4;
            if (j0 + j < N) {
              const f32x16 &c = acc[tm][tn];
              f32x4 *p = (f32x4 *)(o + (size_t)i * N + j);
              f32x4 v = *p;
              v[0] += c[4 * g + 0];
              v[1] += c[4 * g + 1];
              v[2] += c[4 * g + 2];
              v[3] += c[4 * g + 3];
              *p = v;
            }
          }
      }
    }
  }
}

constexpr size_t kGemmLds = 2 * 2 * TILE_ELEMS * sizeof(uint16_t);

// ---------------------------------------------------------------------------------------
// fp32 vector-ALU path (small shapes)
// ---------------------------------------------------------------------------------------

__device__ inline int seg_of_row(const int32_t *cu, int G, int row) {
  int lo = 0, hi = G;  // last rho with cu[rho] <= row
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

template <int OP>
__global__ __launch_bounds__(256) void k_ggemm_f32_rows(const float *__restrict__ a,
                                                        const float *__restrict__ w,
                                                        const int32_t *__restrict__ cu,
                                                        float *__restrict__ out, int G,
                                                        int M_total, int Kd, int N) {
  const int ncols = OP == MOE_GEMM_FWD ? N : Kd;
  const int kc = OP == MOE_GEMM_FWD ? Kd : N;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int row = (int)(idx / ncols), col = (int)(idx % ncols);
  const int end = min(max(cu[G], 0), M_total);
  if (row >= end || row < max(cu[0], 0)) return;
  const int rho = seg_of_row(cu, G, row);
  if (row >= cu[rho + 1]) return;
  const float *wr = w + (size_t)rho * Kd * N;
  const float *ar = a + (size_t)row * kc;
  float s = 0.f;
  for (int c = 0; c < kc; ++c) {
    const float wv = OP == MOE_GEMM_FWD ? wr[(size_t)c * N + col] : wr[(size_t)col * N + c];
    s = __builtin_fmaf(ar[c], wv, s);
  }
  out[(size_t)row * ncols + col] = s;
}

__global__ __launch_bounds__(256) void k_ggemm_f32_wgrad(const float *__restrict__ a,
                                                         const float *__restrict__ bm,
                                                         const int32_t *__restrict__ cu,
                                                         float *__restrict__ out, int G,
                                                         int M_total, int Kd, int N) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long per = (long long)Kd * N;
  if (idx >= per * G) return;
  const int rho = (int)(idx / per);
  const int i = (int)((idx % per) / N), j = (int)(idx % N);
  const int lo = min(max(cu[rho], 0), M_total), hi = min(max(cu[rho + 1], 0), M_total);
  if (hi <= lo) return;
  float s = 0.f;
  for (int m = lo; m < hi; ++m) s = __builtin_fmaf(a[(size_t)m * Kd + i], bm[(size_t)m * N + j], s);
  out[idx] += s;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status_t moe_group_gemm(moe_gemm_op op, moe_dtype dtype, int32_t G,
                                       int32_t M_total, int32_t Kd, int32_t N, const void *a,
                                       const void *b, const int32_t *cu_seqlens, void *out,
                                       hipStream_t stream) {
  if (!a || !b || !cu_seqlens || !out) return MOE_EINVAL;
  if (G < 1 || G > kMaxG || M_total < 0 || Kd < 8 || N < 8 || Kd % 8 || N % 8) return MOE_EINVAL;
  if (op != MOE_GEMM_FWD && op != MOE_GEMM_DGRAD && op != MOE_GEMM_WGRAD) return MOE_EINVAL;
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_EINVAL;
  if ((long long)M_total * (Kd > N ? Kd : N) >= (1LL << 40)) return MOE_EINVAL;
  if (M_total == 0) return MOE_OK;
  if (dtype == MOE_F32) {
    if (op == MOE_GEMM_WGRAD) {
      const long long n = (long long)G * Kd * N;
      hipLaunchKernelGGL(k_ggemm_f32_wgrad, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                         stream, (const float *)a, (const float *)b, cu_seqlens, (float *)out, G,
                         M_total, Kd, N);
    } else {
      const long long n = (long long)M_total * (op == MOE_GEMM_FWD ? N : Kd);
      if (op == MOE_GEMM_FWD)
        hipLaunchKernelGGL(k_ggemm_f32_rows<MOE_GEMM_FWD>, dim3((unsigned)((n + 255) / 256)),
                           dim3(256), 0, stream, (const float *)a, (const float *)b, cu_seqlens,
                           (float *)out, G, M_total, Kd, N);
      else
        hipLaunchKernelGGL(k_ggemm_f32_rows<MOE_GEMM_DGRAD>, dim3((unsigned)((n + 255) / 256)),
                           dim3(256), 0, stream, (const float *)a, (const float *)b, cu_seqlens,
                           (float *)out, G, M_total, Kd, N);
    }
    return launch_status();
  }
  const int grid = device_cu_count();
  switch (op) {
    case MOE_GEMM_FWD:
      hipLaunchKernelGGL(k_ggemm_bf16<MOE_GEMM_FWD>, dim3(grid), dim3(kGemmThreads), kGemmLds,
                         stream, (const uint16_t *)a, (const uint16_t *)b, cu_seqlens, out, G,
                         M_total, Kd, N);
      break;
    case MOE_GEMM_DGRAD:
      hipLaunchKernelGGL(k_ggemm_bf16<MOE_GEMM_DGRAD>, dim3(grid), dim3(kGemmThreads), kGemmLds,
                         stream, (const uint16_t *)a, (const uint16_t *)b, cu_seqlens, out, G,
                         M_total, Kd, N);
      break;
    default:
      hipLaunchKernelGGL(k_ggemm_bf16<MOE_GEMM_WGRAD>, dim3(grid), dim3(kGemmThreads), kGemmLds,
                         stream, (const uint16_t *)a, (const uint16_t *)b, cu_seqlens, out, G,
                         M_total, Kd, N);
  }
  return launch_status();
}

namespace moe {
// Allow the GEMM kernels their full dynamic LDS; called once per device from api.hip.
void gemm_set_attributes() {
  (void)hipFuncSetAttribute((const void *)k_ggemm_bf16<MOE_GEMM_FWD>,
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLds);
  (void)hipFuncSetAttribute((const void *)k_ggemm_bf16<MOE_GEMM_DGRAD>,
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLds);
  (void)hipFuncSetAttribute((const void *)k_ggemm_bf16<MOE_GEMM_WGRAD>,
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLds);
}
}  // namespace moe
