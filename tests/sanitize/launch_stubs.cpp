// Stand-ins for the kernel launchers, linked into the sanitizer build of the
// C ABI's host code (tests/sanitize/api_driver.cpp) in place of the kernel
// sources.  The driver never reaches a launch (every call it makes is refused
// on the host, or is a host-only query), so each launcher reports an error and
// each size helper a plausible value.
#include "csa_backward.hpp"
#include "csa_launch.hpp"

namespace csa {

size_t rows_lds_bytes(int, int, int, int cap) { return 64 * 1024 + (size_t)cap * 8; }
size_t topk_lds_bytes(int cap) { return (size_t)cap * 32; }
size_t topk_block_lds_bytes(int cap, int top_k, int) { return (size_t)cap * 64 + (size_t)top_k * 8; }
size_t topk_block_fast_only_lds_bytes(int, int W) { return (size_t)W * 4 + 16448; }
hipError_t launch_rows(int, int, int, const KernelArgs &, size_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_split(int, int, const KernelArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_stream(int, int, const KernelArgs &, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_topk(const KernelArgs &, size_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_topk_block(const KernelArgs &, size_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_kl_grad(const KernelArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_bwd_rows(int, int, const BwdArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_bwd_keys(int, int, const BwdArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_bwd_reduce(const BwdArgs &, hipStream_t) { return hipErrorNoDevice; }

} // namespace csa
