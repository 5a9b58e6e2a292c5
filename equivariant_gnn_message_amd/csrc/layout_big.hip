// Kernels of the layout 64x(0e+1o+2e), lmax 3 -> 64x(0e+1o+2e+3o).
#include "conv_kernels.h"
#include "conv_mfma.h"

namespace e3c {
namespace {

using L = Layout<64, natural_code(2), 3, natural_code(3)>;
using LS = SenderOrdered<L>;

constexpr LayoutTables kTables = L::T;
constexpr CGValues<L::NNZ> kCG = L::CG;

// Variant 0 of each list is the default (the fastest measured on MI355X for
// the workload of this layout); the others stay selectable for comparison.
const FwdLauncher kF32[] = {launch_fwd_pipe<L, float, 2, 2>, launch_fwd<L, float, 4, 4>, launch_fwd_pipe<L, float, 4, 4>};
// The default runs one wave per work-group (each wave's slot is released as
// soon as it ends): 1.637 against 1.650 ms with four-wave work-groups
// (variant 8) on the large bf16 graph, MI355X.
const FwdLauncher kBF16[] = {launch_fwd_pipe<L, bf16_bits, 2, 2, true, false, false, 1>, launch_fwd<L, bf16_bits, 4, 4>,
                             launch_fwd_pipe<L, bf16_bits, 4, 4>, launch_fwd_pipe<L, bf16_bits, 4, 2>,
                             launch_fwd_pipe<L, bf16_bits, 2, 1>, launch_fwd_pipe<L, bf16_bits, 2, 2>,
                             launch_fwd_mfma<L, false>, launch_fwd_mfma<L, true>,
                             launch_fwd_pipe<L, bf16_bits, 2, 2, true>};
const BwdLauncher kBwd[] = {launch_bwd<L, 2, 2>, launch_bwd_pipe<L, 2, 2>};

const FwdLauncher kSenderF32[] = {launch_fwd_pipe<LS, float, 2, 2>};
const FwdLauncher kSenderBF16[] = {launch_fwd_pipe<LS, bf16_bits, 2, 2, true>};
const BwdLauncher kSenderBwd[] = {launch_bwd<LS, 2, 2>};

#define E3C_N(a) (int)(sizeof(a) / sizeof((a)[0]))

}  // namespace

const KernelSet* kernels_big() {
  static const KernelSet k = {
    L::C, L::XCODE, L::L, L::OCODE, &kTables, kCG.v,
    {kF32, E3C_N(kF32), kBF16, E3C_N(kBF16), kBwd, E3C_N(kBwd), launch_bwd_pipe<L, 2, 2, true>,
     launch_jvp<L, float, 2, 2>, launch_jvp_pipe<L, bf16_bits, 2, 2, false, 1>, nullptr,
     launch_bwd_pairs<L, 1, 16>, launch_fwd_pipe<L, float, 2, 2, false, true>,
     launch_fwd_pipe<L, bf16_bits, 2, 2, true, true>, launch_fwd_pipe<L, float, 2, 2, false, false, true>},
    {kSenderF32, 1, kSenderBF16, 1, kSenderBwd, 1, launch_bwd_pipe<LS, 2, 2, true>,
     launch_jvp<LS, float, 2, 2>, launch_jvp_pipe<LS, bf16_bits, 2, 2, false>},
  };
  return &k;
}

}  // namespace e3c
