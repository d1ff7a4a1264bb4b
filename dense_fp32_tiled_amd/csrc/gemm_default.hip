// gemm_default.hip -- the default fp32 kernel's 16-byte form, alone in its
// translation unit (see default_config.hpp).
#include "default_config.hpp"

namespace dft {

hipError_t launch_default_vec4(const Args& a, Split sp, hipStream_t stream) {
    return launch_mfma<Mfma256x256Bk32Pipe<4>>(a, sp, stream);
}

}  // namespace dft
