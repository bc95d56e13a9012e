// Kernel instantiations for dtype f16_f32 (inputs F16, output F32).
#include "gemm_streamk.hpp"
#include "configs.def"
#include "gemm_strip.hpp"

namespace mg {

#define MG_ENTRY(BM, BN, BK, WM, WN, MI, SWZ)                                        \
    {"f16_f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s2" MG_SWZNAME_##SWZ, \
     BM, BN, BK, WM, WN, MI, SWZ,                                                  \
     &Inst<In::F16, Out::F32, BM, BN, BK, WM, WN, MI, SWZ>::launch, 2, false},

#define MG_DMA_ENTRY(BM, BN, BK, WM, WN, MI, ST)                                      \
    {"f16_f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s" #ST " dma",          \
     BM, BN, BK, WM, WN, MI, true,                                                  \
     &DmaInst<In::F16, Out::F32, BM, BN, BK, WM, WN, MI, ST>::launch, ST, true},

#define MG_DMA_SK_ENTRY(BM, BN, BK, WM, WN, MI, ST, OCC)                              \
    {"f16_f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s" #ST " dma sk",       \
     BM, BN, BK, WM, WN, MI, true,                                                  \
     &Dma16SkInst<In::F16, Out::F32, BM, BN, BK, WM, WN, MI, ST>::launch, ST, true, OCC},

#define MG_SCALAR_ENTRY(BM, BN, BK, WM, WN, MI)                                        \
    {"f16_f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s2 swz scalar",              \
     BM, BN, BK, WM, WN, MI, true, &Inst<In::F16, Out::F32, BM, BN, BK, WM, WN, MI, true, false>::launch, 2, false, 0, true},

#define MG_DMA2_ENTRY(BM, BN, BK, WM, WN, MI, SA, SB)                                  \
    {"f16_f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s" #SA "x" #SB " dma",        \
     BM, BN, BK, WM, WN, MI, true,                                                  \
     &DmaInst<In::F16, Out::F32, BM, BN, BK, WM, WN, MI, SA, SB>::launch, SA, true},

#define MG_PP_ENTRY(BM, BN, BK, WM, WN, MI)                                          \
    {"f16_f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s3x2 pp",                  \
     BM, BN, BK, WM, WN, MI, true,                                                  \
     &PpInst<In::F16, Out::F32, BM, BN, BK, WM, WN, MI>::launch, 3, true, 0, false, true},

#define MG_DMA_SPLIT_ENTRY(BM, BN, BK, WM, WN, MI, SA, SB, OCC)                       \
    {"f16_f32 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s" #SA "x" #SB " dma split",       \
     BM, BN, BK, WM, WN, MI, true,                                                  \
     &Dma16SplitInst<In::F16, Out::F32, BM, BN, BK, WM, WN, MI, SA, SB>::launch, SA, true, 0, false, false, OCC},

static const KernelEntry kEntries[] = {MG_CONFIGS_16(MG_ENTRY) MG_DMA_CONFIGS_16(MG_DMA_ENTRY)
                                           MG_DMA_SK_CONFIGS_16(MG_DMA_SK_ENTRY)
                                           MG_SCALAR_CONFIGS_16(MG_SCALAR_ENTRY)
                                               MG_DMA2_CONFIGS_16(MG_DMA2_ENTRY)
                                                   MG_PP_CONFIGS_16(MG_PP_ENTRY)
                                                       MG_DMA_SPLIT_CONFIGS_16(MG_DMA_SPLIT_ENTRY)};

hipError_t strip_f16_f32(int layout, bool rows, const Params& p, hipStream_t s)
{
    return StripInst<In::F16, Out::F32>::launch(layout, rows, p, s);
}

const KernelEntry* entries_f16_f32(int* n)
{
    *n = (int)(sizeof(kEntries) / sizeof(kEntries[0]));
    return kEntries;
}

}  // namespace mg
