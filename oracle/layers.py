"""Layer pattern of the Gemma 4 hybrid stack.

Test infrastructure only (see ``oracle/__init__``).

pegainfer "Gemma 4" page, intro: five of every six layers are sliding-window
local layers; every sixth layer, and the last one, is global.  Architecture
notes table: the 12B line has 48 layers, 8 global and 40 local.
"""

from __future__ import annotations


def is_global(layer: int, num_layers: int) -> bool:
    """Layer i (0-based) is global iff it is a sixth layer or the last one."""
    return (layer + 1) % 6 == 0 or layer == num_layers - 1


def global_layers(num_layers: int) -> list[int]:
    return [i for i in range(num_layers) if is_global(i, num_layers)]
