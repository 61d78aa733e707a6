// Kernel instances for fp16 (IEEE binary16) data.
#include "fnorm_instances.hpp"

namespace fnorm {
void register_f16(std::vector<Variant>& table) { register_dtype<DT_F16>(table); }
}  // namespace fnorm
