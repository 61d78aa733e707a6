// Kernel instances for fp32 data.
#include "fnorm_instances.hpp"

namespace fnorm {
void register_f32(std::vector<Variant>& table) { register_dtype<DT_F32>(table); }
}  // namespace fnorm
