// Host-only stand-ins for libkvc's kernel launchers, so that the host side of
// kvc_api.hip (argument validation, workspace layout, dispatch) can be built
// with AddressSanitizer / UndefinedBehaviorSanitizer and driven on a machine
// without a GPU.  Each stub only counts its calls; nothing is launched.
#include "kvc_internal.h"

namespace kvc {

int g_stub_launches = 0;

hipError_t launch_attn(const AttnArgs &, int, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_split(const AttnArgs &, bool, int, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_accumulate(const AccumArgs &, int, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_prompt_scores(const PromptArgs &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_select(const SelectArgs &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_compact(const CompactArgs &, int, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_kivi_prefill(const KiviArgs &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_kivi_decode(const KiviArgs &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_step_split(const AttnArgs &, const SelectArgs &, const CompactArgs &, int,
                             hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_fused(const FusedArgs &, int, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_stream_read(const void *, size_t, uint32_t *, hipStream_t) { ++g_stub_launches; return hipSuccess; }
// the prompt-scoring workspace: one fp32 log-sum-exp per query row and head
size_t prompt_workspace_bytes(int units, int m_rows, int G) {
    return (size_t)units * (size_t)m_rows * (size_t)G * sizeof(float);
}

}  // namespace kvc

extern "C" int kvc_stub_launches(void) { return kvc::g_stub_launches; }
