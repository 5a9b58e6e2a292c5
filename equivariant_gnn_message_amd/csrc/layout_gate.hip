// Kernels of the layout 32x0e+32x1o, lmax 3 -> 32x(0e+1o+2e).
#include "conv_kernels.h"
#include "conv_radial.h"

namespace e3c {
namespace {

using L = Layout<32, natural_code(1), 3, natural_code(2)>;
using LS = SenderOrdered<L>;

constexpr LayoutTables kTables = L::T;
constexpr CGValues<L::NNZ> kCG = L::CG;

// Variant 0 of each list is the default (the fastest measured on MI355X for
// the workload of this layout); the others stay selectable for comparison.
// The default runs one wave per work-group: 21.8 against 22.3 us with four
// waves per work-group (variant 5) on the gate-points graph, MI355X.
const FwdLauncher kF32[] = {launch_fwd_pipe<L, float, 4, 4, true, false, false, 1>, launch_fwd<L, float, 4, 4>,
                            launch_fwd_pipe<L, float, 4, 2>, launch_fwd_pipe<L, float, 2, 2>,
                            launch_fwd_pipe<L, float, 4, 4>, launch_fwd_pipe<L, float, 4, 4, true>};
const FwdLauncher kBF16[] = {launch_fwd_pipe<L, bf16_bits, 4, 4>, launch_fwd<L, bf16_bits, 4, 4>};
const BwdLauncher kBwd[] = {launch_bwd<L, 2, 4>, launch_bwd<L, 1, 2>, launch_bwd_pipe<L, 2, 4>};

const FwdLauncher kSenderF32[] = {launch_fwd_pipe<LS, float, 4, 4>};
const FwdLauncher kSenderBF16[] = {launch_fwd_pipe<LS, bf16_bits, 4, 4>};
const BwdLauncher kSenderBwd[] = {launch_bwd<LS, 2, 4>};

#define E3C_N(a) (int)(sizeof(a) / sizeof((a)[0]))

}  // namespace

const KernelSet* kernels_gate() {
  static const KernelSet k = {
    L::C, L::XCODE, L::L, L::OCODE, &kTables, kCG.v,
    {kF32, E3C_N(kF32), kBF16, E3C_N(kBF16), kBwd, E3C_N(kBwd), launch_bwd_pipe<L, 2, 4, true>,
     launch_jvp<L, float, 2, 4>, launch_jvp<L, bf16_bits, 2, 4>, launch_fwd_radial<L>,
     launch_bwd_pairs<L, 2, 16>, launch_fwd_pipe<L, float, 4, 4, true, true>,
     launch_fwd_pipe<L, bf16_bits, 4, 4, false, true>, launch_fwd_pipe<L, float, 4, 4, true, false, true>},
    {kSenderF32, 1, kSenderBF16, 1, kSenderBwd, 1, launch_bwd_pipe<LS, 2, 4, true>,
     launch_jvp<LS, float, 2, 4>, launch_jvp<LS, bf16_bits, 2, 4>},
  };
  return &k;
}

}  // namespace e3c
