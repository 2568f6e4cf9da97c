"""CPU oracle (test infrastructure only; see lora_oracle's header)."""
from .lora_oracle import *  # noqa: F401,F403
from .lora_oracle import __all__  # noqa: F401
