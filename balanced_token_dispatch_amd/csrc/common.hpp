// Shared device and host helpers of libmoe.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kWave = 64;

// Plan blob word offsets (see moe_plan in moe.h).
struct PlanLayout {
  int E, R, B;
  int off_T, off_keep, off_rep_first, off_rep_n;
  int off_rexp, off_rrank, off_rslot, off_rstart, off_rcount;
  int off_sexp, off_sstart, off_scount, words;
  __host__ __device__ PlanLayout(int E_, int R_, int B_) : E(E_), R(R_), B(B_) {
    const int L = E + R;
    off_T = 8;
    off_keep = off_T + E;
    off_rep_first = off_keep + E;
    off_rep_n = off_rep_first + E;
    off_rexp = off_rep_n + E;
    off_rrank = off_rexp + L;
    off_rslot = off_rrank + L;
    off_rstart = off_rslot + L;
    off_rcount = off_rstart + L;
    off_sexp = off_rcount + L;
    off_sstart = off_sexp + R * B;
    off_scount = off_sstart + R * B;
    words = off_scount + R * B;
  }
};

// fp32 -> bf16 bits, IEEE round to nearest even (hardware v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Host-side validation of moe_dims against the limits stated in moe.h.
inline bool dims_ok(const moe_dims *d) {
  if (!d) return false;
  if (d->R < 1 || d->R > 512 || d->S < 1 || d->K < 1 || d->E < 1 || d->E > 1024) return false;
  if (d->E % d->R != 0 || d->K > d->E || d->B < 0 || d->B > 64) return false;
  const long long copies = (long long)d->R * d->S * d->K;
  if (copies >= (1LL << 31)) return false;
  return true;
}

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

inline moe_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int device_cu_count();  // cached per device, in api.hip

}  // namespace moe
