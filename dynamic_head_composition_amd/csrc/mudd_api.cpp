// C ABI of MUDD layer mixing: argument validation and dispatch.  Validation
// happens before any HIP call, so every error path runs without a GPU.
#include "../../include/mudd.h"

#include <hip/hip_runtime.h>

#include "mudd_internal.h"

static_assert(MUDD_MAX_STREAMS == mudd::kMaxJ && MUDD_MAX_WAYS == mudd::kMaxW, "limits");

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_sizes(int dtype, int64_t T, int dm, int W, int J) {
  if (dtype != LDC_BF16 && dtype != LDC_F32) return LDC_ERR_DTYPE;
  if (T < 0 || W < 1 || W > MUDD_MAX_WAYS || J < 1 || J > MUDD_MAX_STREAMS) return LDC_ERR_SHAPE;
  if (dm < 4 || dm > MUDD_MAX_DIM || dm % 4 != 0) return LDC_ERR_SHAPE;
  if (T > ((int64_t)1 << 40) / dm) return LDC_ERR_SHAPE;
  return LDC_OK;
}

// n device pointers from a host array: present and 16-byte aligned
template <typename P>
int check_ptrs(const P* arr, int n) {
  if (arr == nullptr) return LDC_ERR_NULL;
  for (int i = 0; i < n; ++i)
    if (arr[i] == nullptr) return LDC_ERR_NULL;
  for (int i = 0; i < n; ++i)
    if (!aligned16(arr[i])) return LDC_ERR_ALIGN;
  return LDC_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? LDC_OK : LDC_ERR_HIP; }

}  // namespace

extern "C" {

int mudd_fwd(int dtype, int64_t T, int dm, int W, int J, const void* const* xs, const float* a,
             float* const* ys, void* stream) {
  int st = check_sizes(dtype, T, dm, W, J);
  if (st != LDC_OK) return st;
  if (a == nullptr) return LDC_ERR_NULL;
  if ((st = check_ptrs(xs, J)) != LDC_OK) return st;
  if ((st = check_ptrs(ys, W)) != LDC_OK) return st;
  if (!aligned16(a)) return LDC_ERR_ALIGN;
  if (T == 0) return LDC_OK;
  mudd::FwdArgs args{};
  for (int j = 0; j < J; ++j) args.x[j] = xs[j];
  for (int w = 0; w < W; ++w) args.y[w] = ys[w];
  args.a = a;
  args.T = T;
  args.dm = dm;
  args.W = W;
  args.J = J;
  return launch_status(mudd::fwd_dispatch(dtype, args, static_cast<hipStream_t>(stream)));
}

int mudd_bwd(int dtype, int64_t T, int dm, int W, int J, const void* const* xs, const float* a,
             const void* const* dys, float* const* dxs, float* da, void* stream) {
  int st = check_sizes(dtype, T, dm, W, J);
  if (st != LDC_OK) return st;
  if (a == nullptr || da == nullptr) return LDC_ERR_NULL;
  if ((st = check_ptrs(xs, J)) != LDC_OK) return st;
  if ((st = check_ptrs(dys, W)) != LDC_OK) return st;
  if ((st = check_ptrs(dxs, J)) != LDC_OK) return st;
  if (!aligned16(a) || !aligned16(da)) return LDC_ERR_ALIGN;
  if (T == 0) return LDC_OK;
  mudd::BwdArgs args{};
  for (int j = 0; j < J; ++j) {
    args.x[j] = xs[j];
    args.dx[j] = dxs[j];
  }
  for (int w = 0; w < W; ++w) args.dy[w] = dys[w];
  args.a = a;
  args.da = da;
  args.T = T;
  args.dm = dm;
  args.W = W;
  args.J = J;
  return launch_status(mudd::bwd_dispatch(dtype, args, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
