// Stand-ins for the device-side launchers (kernels.hip, swap.hip,
// scratch.hip) in the host-only sanitizer build of the library
// (tests/test_host_sanitized.py): host-only pools never reach them, and
// each one fails loudly if it is reached.
#include <cstdio>
#include <cstdlib>

#include "kernels.hpp"
#include "scratch.hpp"
#include "swap.hpp"

namespace pa {
namespace {
[[noreturn]] void unreachable(const char* what) {
  std::fprintf(stderr, "host-only build: %s reached\n", what);
  std::abort();
}
}  // namespace

hipError_t launch_append(const AppendParams&, const InlineMeta*, hipStream_t) { unreachable("launch_append"); }
hipError_t launch_attention(DType, const AttnParams&, const InlineMeta*, hipStream_t) {
  unreachable("launch_attention");
}
hipError_t launch_merge(DType, const AttnParams&, hipStream_t) { unreachable("launch_merge"); }
hipError_t launch_prefix(DType, const AttnParams&, hipStream_t) { unreachable("launch_prefix"); }
int prefix_rows_per_unit(int, int) { unreachable("prefix_rows_per_unit"); }
int prefix_units_per_cu(int, int) { unreachable("prefix_units_per_cu"); }
bool prefix_in_attention_launch(int, int, int) { unreachable("prefix_in_attention_launch"); }
int append_blocks64(const AppendParams&) { unreachable("append_blocks64"); }
int append_blocks_prefix_launch(const AppendParams&) { unreachable("append_blocks_prefix_launch"); }
hipError_t launch_merge_rows(DType, const AttnParams&, hipStream_t) { unreachable("launch_merge_rows"); }
int merge_rows_workgroups(const AttnParams&) { unreachable("merge_rows_workgroups"); }
int prefix_launch_waves() { unreachable("prefix_launch_waves"); }
int prefix_rows_per_wave(int) { unreachable("prefix_rows_per_wave"); }
int max_rows_for_head_dim(int) { unreachable("max_rows_for_head_dim"); }
int tile_rows_for_call(int, int, int) { unreachable("tile_rows_for_call"); }
hipError_t launch_swap(const SwapParams&, hipStream_t) { unreachable("launch_swap"); }
hipError_t scratch_address(int, char**) { unreachable("scratch_address"); }
hipError_t launch_words(int32_t*, const InlineMeta&, int, uint32_t*, int, hipStream_t) {
  unreachable("launch_words");
}
}  // namespace pa
