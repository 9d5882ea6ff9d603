// A kernel that returns at once, launched with the grid shape of a path
// kernel: its duration in a kernel trace is the launch floor of that shape
// (workgroup dispatch, wave start and retirement, the cache maintenance at the
// kernel boundaries), against which the path kernels' durations are read.
#include "launchers.h"

namespace dsa {

template <int NT>
__global__ __launch_bounds__(NT) void launch_floor_kernel() {}

int launch_floor(int workgroups, int threads, hipStream_t stream) {
  switch (threads) {
    case 256:
      hipLaunchKernelGGL(launch_floor_kernel<256>, dim3(workgroups), dim3(256), 0, stream);
      break;
    case 512:
      hipLaunchKernelGGL(launch_floor_kernel<512>, dim3(workgroups), dim3(512), 0, stream);
      break;
    default:
      hipLaunchKernelGGL(launch_floor_kernel<1024>, dim3(workgroups), dim3(1024), 0, stream);
      break;
  }
  return 0;
}

}  // namespace dsa
