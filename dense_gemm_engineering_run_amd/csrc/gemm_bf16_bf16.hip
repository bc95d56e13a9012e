// Kernel instantiations for dtype bf16_bf16 (inputs BF16, output BF16).
#include "gemm_streamk.hpp"
#include "configs.def"
#include "gemm_strip.hpp"

namespace mg {

#define MG_ENTRY(BM, BN, BK, WM, WN, MI, SWZ)                                        \
    {"bf16_bf16 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s2" MG_SWZNAME_##SWZ, \
     BM, BN, BK, WM, WN, MI, SWZ,                                                  \
     &Inst<In::BF16, Out::BF16, BM, BN, BK, WM, WN, MI, SWZ>::launch, 2, false},

#define MG_DMA_ENTRY(BM, BN, BK, WM, WN, MI, ST)                                      \
    {"bf16_bf16 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s" #ST " dma",          \
     BM, BN, BK, WM, WN, MI, true,                                                  \
     &DmaInst<In::BF16, Out::BF16, BM, BN, BK, WM, WN, MI, ST>::launch, ST, true},

#define MG_DMA_SK_ENTRY(BM, BN, BK, WM, WN, MI, ST, OCC)                              \
    {"bf16_bf16 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s" #ST " dma sk",       \
     BM, BN, BK, WM, WN, MI, true,                                                  \
     &Dma16SkInst<In::BF16, Out::BF16, BM, BN, BK, WM, WN, MI, ST>::launch, ST, true, OCC},

#define MG_SCALAR_ENTRY(BM, BN, BK, WM, WN, MI)                                        \
    {"bf16_bf16 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s2 swz scalar",              \
     BM, BN, BK, WM, WN, MI, true, &Inst<In::BF16, Out::BF16, BM, BN, BK, WM, WN, MI, true, false>::launch, 2, false, 0, true},

#define MG_DMA2_ENTRY(BM, BN, BK, WM, WN, MI, SA, SB)                                  \
    {"bf16_bf16 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s" #SA "x" #SB " dma",        \
     BM, BN, BK, WM, WN, MI, true,                                                  \
     &DmaInst<In::BF16, Out::BF16, BM, BN, BK, WM, WN, MI, SA, SB>::launch, SA, true},

#define MG_PP_ENTRY(BM, BN, BK, WM, WN, MI)                                          \
    {"bf16_bf16 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s3x2 pp",                  \
     BM, BN, BK, WM, WN, MI, true,                                                  \
     &PpInst<In::BF16, Out::BF16, BM, BN, BK, WM, WN, MI>::launch, 3, true, 0, false, true},

#define MG_DMA_SPLIT_ENTRY(BM, BN, BK, WM, WN, MI, SA, SB, OCC)                       \
    {"bf16_bf16 " #BM "x" #BN "x" #BK " w" #WM "x" #WN " mfma" #MI " s" #SA "x" #SB " dma split",       \
     BM, BN, BK, WM, WN, MI, true,                                                  \
     &Dma16SplitInst<In::BF16, Out::BF16, BM, BN, BK, WM, WN, MI, SA, SB>::launch, SA, true, 0, false, false, OCC},

static const KernelEntry kEntries[] = {MG_CONFIGS_16(MG_ENTRY) MG_DMA_CONFIGS_16(MG_DMA_ENTRY)
                                           MG_DMA_SK_CONFIGS_16(MG_DMA_SK_ENTRY)
                                           MG_SCALAR_CONFIGS_16(MG_SCALAR_ENTRY)
                                               MG_DMA2_CONFIGS_16(MG_DMA2_ENTRY)
                                                   MG_PP_CONFIGS_16(MG_PP_ENTRY)
                                                       MG_DMA_SPLIT_CONFIGS_16(MG_DMA_SPLIT_ENTRY)};

hipError_t strip_bf16_bf16(int layout, bool rows, const Params& p, hipStream_t s)
{
    return StripInst<In::BF16, Out::BF16>::launch(layout, rows, p, s);
}

const KernelEntry* entries_bf16_bf16(int* n)
{
    *n = (int)(sizeof(kEntries) / sizeof(kEntries[0]));
    return kEntries;
}

}  // namespace mg
