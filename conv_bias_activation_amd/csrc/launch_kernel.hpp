// launch_kernel.hpp — every kernel of the library is queued through
// launch_kernel(), which takes the refusal (if any) from hipLaunchKernel's own
// return value.  hipGetLastError() would also report an error that some
// unrelated earlier runtime call left on the thread.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <tuple>
#include <utility>

namespace biasact {

// First launch refusal since the calling thread last cleared it (api.hip
// clears it before each entry point's launches).
extern thread_local hipError_t t_launch_error;

// Description of the main kernel the calling thread queued last (reported by
// biasact_last_tile_config).
constexpr int kLaunchDescBytes = 96;
extern thread_local char t_launch_desc[kLaunchDescBytes];

inline void note_launch(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(t_launch_desc, sizeof(t_launch_desc), fmt, ap);
  va_end(ap);
}

template <class... P, size_t... I>
inline hipError_t launch_argv(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s,
                              std::tuple<P...>& t, std::index_sequence<I...>) {
  void* argv[] = {static_cast<void*>(&std::get<I>(t))...};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, 0, s);
}

// k<<<grid, block, 0, s>>>(args...), with the arguments converted to the
// kernel's parameter types.
template <class... P, class... A>
inline void launch_kernel(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> t(std::forward<A>(args)...);
  const hipError_t e = launch_argv(k, grid, block, s, t, std::index_sequence_for<P...>{});
  if (e != hipSuccess && t_launch_error == hipSuccess) t_launch_error = e;
}

}  // namespace biasact
