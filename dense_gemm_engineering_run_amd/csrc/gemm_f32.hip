// Kernel instantiations for dtype f32 (inputs F32, output F32).
#include "gemm_kernel.hpp"
#include "configs.def"

namespace mg {

#define MG_ENTRY(BM, BN, BK, WM, WN, MI, SWZ)                                        \
    {"f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s2" MG_SWZNAME_##SWZ, \
     BM, BN, BK, WM, WN, MI, SWZ,                                                  \
     &Inst<In::F32, Out::F32, BM, BN, BK, WM, WN, MI, SWZ>::launch, 2, false},

static const KernelEntry kEntries[] = {MG_CONFIGS_F32(MG_ENTRY)};

const KernelEntry* entries_f32(int* n)
{
    *n = (int)(sizeof(kEntries) / sizeof(kEntries[0]));
    return kEntries;
}

}  // namespace mg
