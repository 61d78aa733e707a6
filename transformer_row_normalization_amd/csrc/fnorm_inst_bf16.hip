// Kernel instances for bf16 data.
#include "fnorm_instances.hpp"

namespace fnorm {
void register_bf16(std::vector<Variant>& table) { register_dtype<DT_BF16>(table); }
}  // namespace fnorm
