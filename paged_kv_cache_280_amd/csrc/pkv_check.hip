// Check of the table contract on the device.  The attention kernels clamp block
// ids and lengths into range instead of checking them (no memory outside the
// pools is read), so a caller whose tables break the contract gets meaningless
// rows without an error; this check names the first sequence that does.  The
// contract is the block-table walk of "PagedAttention (vLLM)" (troisinh.com,
// section "Cơ chế Block Table"): position t of sequence s lives in the block
// that entry t / B of its row names, so the first ceil(L / B) entries of a row
// must be blocks of the pool.
//
// One wave per sequence; a violation is reported as 4 * s + kind through an
// unsigned atomic minimum on a word that a first one-thread kernel resets to
// 0xFFFFFFFF (no memset, so the pair can be captured in a graph).

#include "pkv_internal.h"

namespace pkv {
namespace {

__global__ void check_reset_kernel(uint32_t* result) { *result = 0xFFFFFFFFu; }

__global__ __launch_bounds__(kWave* kWavesPerGroup) void check_kernel(
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ qlens, uint32_t* result, CheckDims c) {
  const int lane = __lane_id();
  const int64_t s = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + threadIdx.x / kWave;
  if (s >= c.S) return;
  const int32_t cap = c.M * c.B;  // positions one table row can address
  const int32_t L = lens[s];
  uint32_t kind = 0;
  if (L < 0 || L > cap) kind = 1;
  // entries the attention kernels read: those of the clamped length
  const int32_t Lc = L < 0 ? 0 : (L > cap ? cap : L);
  const int32_t nblk = (Lc + c.B - 1) / c.B;
  bool bad = false;
  for (int32_t j = lane; j < nblk; j += kWave) {
    const int32_t b = tables[s * c.M + j];
    bad = bad || b < 0 || b >= c.NB;
  }
  if (kind == 0 && __ballot(bad) != 0) kind = 2;
  if (kind == 0 && qlens != nullptr) {
    const int32_t T = qlens[s];
    if (T < 0 || T > Lc || T > c.Qmax) kind = 3;
  }
  if (kind != 0 && lane == 0) atomicMin(result, static_cast<uint32_t>(4 * s) + kind);
}

}  // namespace

hipError_t launch_check(const int32_t* tables, const int32_t* lens, const int32_t* qlens,
                        int32_t* result, const CheckDims& c, hipStream_t stream) {
  uint32_t* r = reinterpret_cast<uint32_t*>(result);
  hipLaunchKernelGGL(check_reset_kernel, dim3(1), dim3(1), 0, stream, r);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const int64_t groups = (static_cast<int64_t>(c.S) + kWavesPerGroup - 1) / kWavesPerGroup;
  if (groups > 0)
    hipLaunchKernelGGL(check_kernel, dim3(static_cast<uint32_t>(groups)),
                       dim3(kWave * kWavesPerGroup), 0, stream, tables, lens, qlens, r, c);
  return hipGetLastError();
}

}  // namespace pkv
