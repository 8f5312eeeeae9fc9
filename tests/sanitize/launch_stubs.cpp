// Host-only stand-ins for the library's kernel launchers and device queries,
// for the AddressSanitizer / UndefinedBehaviorSanitizer build of api.cpp: the
// host logic (validation, planning, metadata updates) runs instrumented, and
// every path that would reach the GPU ends in hipErrorNoDevice.
#include "../../chunk_causal_dit_wf_amd/csrc/wf_internal.h"
#include "../../chunk_causal_dit_wf_amd/csrc/copy_ref.h"

namespace wf {
hipError_t launch_append(const AppendParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_quant_append(const QuantAppendParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_poison(const PoisonParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_stream_copy(const void*, void*, int64_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_bf16_dma(const AttnParams&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_fp8_dma(const AttnParams&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t attn_fp8_resident_blocks(int, int*) { return hipErrorNoDevice; }
hipError_t launch_attn_merge(const AttnParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t attn_dma_resident_blocks(int, int*) { return hipErrorNoDevice; }
hipError_t launch_attn_bf16_staged(const AttnParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_f32(const AttnParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_fp8kv(const AttnParams&, int, hipStream_t) { return hipErrorNoDevice; }
}  // namespace wf
