// Launcher stand-ins for the host-only sanitizer build of the C-ABI glue: the
// argument checks under test return before any launch, so none of these may
// run (each aborts if it does).
#include <stdio.h>
#include <stdlib.h>

#include "kvq_internal.h"

namespace kvq {

[[noreturn]] static void reached(const char* what) {
  fprintf(stderr, "launcher reached in a validation-only build: %s\n", what);
  abort();
}

hipError_t launch_flush_keys(const CacheView&, const AppendInputs&, int, hipStream_t) { reached("flush"); }
hipError_t launch_append_tokens(const CacheView&, const AppendInputs&, int, hipStream_t) { reached("append"); }
hipError_t launch_update_lengths(const CacheView&, const AppendInputs&, hipStream_t) { reached("lengths"); }
hipError_t launch_append_decode(const CacheView&, const AppendInputs&, hipStream_t) { reached("decode append"); }
hipError_t launch_dequantize(const CacheView&, uint16_t*, uint16_t*, hipStream_t) { reached("dequantize"); }
hipError_t launch_decode_attention(const CacheView&, const AttnPlan&, const uint16_t*, float*, float*,
                                   hipStream_t) { reached("attention"); }
int attention_blocks_per_cu(const CacheView&, int, int) { reached("occupancy"); }

}  // namespace kvq
