// Kernel instantiations for dtype f32 (inputs F32, output F32).
#include "gemm_f32dma.hpp"
#include "configs.def"
#include "gemm_strip.hpp"

namespace mg {

#define MG_ENTRY(BM, BN, BK, WM, WN, MI, SWZ)                                        \
    {"f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s2" MG_SWZNAME_##SWZ, \
     BM, BN, BK, WM, WN, MI, SWZ,                                                  \
     &Inst<In::F32, Out::F32, BM, BN, BK, WM, WN, MI, SWZ>::launch, 2, false},

#define MG_F32DMA_ENTRY(BM, BN, BK, WM, WN, ST)                                      \
    {"f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma32 s" #ST " dma",               \
     BM, BN, BK, WM, WN, 32, true, &F32DmaInst<Out::F32, BM, BN, BK, WM, WN, ST>::launch, ST, true},

#define MG_F32DMA_SK_ENTRY(BM, BN, BK, WM, WN, ST, OCC)                               \
    {"f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma32 s" #ST " dma sk",            \
     BM, BN, BK, WM, WN, 32, true, &F32DmaInst<Out::F32, BM, BN, BK, WM, WN, ST, true>::launch, ST, true, OCC},

#define MG_F32DMA_SCALAR_ENTRY(BM, BN, BK, WM, WN, ST)                               \
    {"f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma32 s" #ST " dma scalar",        \
     BM, BN, BK, WM, WN, 32, true,                                                  \
     &F32DmaInst<Out::F32, BM, BN, BK, WM, WN, ST, false, false>::launch, ST, true, 0, true},

#define MG_SCALAR_ENTRY(BM, BN, BK, WM, WN, MI)                                        \
    {"f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s2 swz scalar",              \
     BM, BN, BK, WM, WN, MI, true, &Inst<In::F32, Out::F32, BM, BN, BK, WM, WN, MI, true, false>::launch, 2, false, 0, true},

#define MG_F32DMA_SPLIT_ENTRY(BM, BN, BK, WM, WN, ST, OCC)                            \
    {"f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma32 s" #ST " dma split",         \
     BM, BN, BK, WM, WN, 32, true, &F32DmaSplitInst<Out::F32, BM, BN, BK, WM, WN, ST>::launch, ST, true, \
     0, false, false, OCC},

static const KernelEntry kEntries[] = {MG_CONFIGS_F32(MG_ENTRY) MG_F32DMA_CONFIGS(MG_F32DMA_ENTRY)
                                           MG_F32DMA_SK_CONFIGS(MG_F32DMA_SK_ENTRY)
                                           MG_F32DMA_SCALAR_CONFIGS(MG_F32DMA_SCALAR_ENTRY)
                                           MG_SCALAR_CONFIGS_F32(MG_SCALAR_ENTRY)
                                               MG_F32DMA_SPLIT_CONFIGS(MG_F32DMA_SPLIT_ENTRY)};

hipError_t strip_f32(int layout, bool rows, const Params& p, hipStream_t s)
{
    return StripInst<In::F32, Out::F32>::launch(layout, rows, p, s);
}

const KernelEntry* entries_f32(int* n)
{
    *n = (int)(sizeof(kEntries) / sizeof(kEntries[0]));
    return kEntries;
}

}  // namespace mg
